/*
 * frnn.h -- C ABI of the MI355X (gfx950) head-wise LSTM / Elman / GRU forward-recurrence library.
 *
 * What is computed (FlashRNN usage example, hottg.com/neural/9889; cell equations of
 * "5.3 LSTM", developnotes.readthedocs.io operator.html, applied per head):
 *
 *   for every batch row b and head n, for t = 0 .. T-1, with h, c the state after step t-1:
 *     pre[g][e] = Wx[b,t,g,n,e] + sum_d h[d] * R[g,n,d,e] + bias[g,n,e]
 *     LSTM  (G = 4 gates i, f, z, o; S = 2 states h, c):
 *        i = sigmoid(pre[0]), f = sigmoid(pre[1]), z = tanh(pre[2]), o = sigmoid(pre[3])
 *        c = f * c + i * z;   h = o * tanh(c)
 *     Elman (G = 1, S = 1):   h = tanh(pre[0])
 *     GRU   (G = 3 gates r, z, n; S = 1): the FlashRNN page names the cell without equations;
 *        this is the textbook form in which the reset gate scales the candidate's recurrent part
 *        after the product, so the n gate keeps Wx apart:
 *        a[g][e] = sum_d h[d] * R[g,n,d,e]
 *        r = sigmoid(Wx[0] + a[0] + bias[0]), z = sigmoid(Wx[1] + a[1] + bias[1])
 *        n = tanh(Wx[2] + r * (a[2] + bias[2])),   h = (1 - z) * n + z * h
 *        (Wx carries the input-side terms and their biases, bias the recurrent-side ones)
 *     states[0,b,t,n,:] = h;  (LSTM) states[1,b,t,n,:] = c
 *   last_states[:,b,0,n,:] = the state after the last step (T == 0: the initial state).
 *
 * Every step uses the complete h of the previous step (synchronous update); batch rows and heads
 * never interact.
 *
 * Conventions shared by every entry point:
 *  - frnn_init() prepares the current device once (the only call that allocates device memory or
 *    waits for the device, apart from frnn_check). Every compute entry point (frnn_fwd, frnn_bwd,
 *    frnn_lstm_stack_fwd, frnn_lstm_stack_bwd) only enqueues kernels: it never allocates, frees or
 *    synchronises, so it may be called under stream capture. On a device frnn_init() has not
 *    prepared it returns FRNN_ENOINIT.
 *  - All tensor arguments are DEVICE pointers owned by the caller. Work is enqueued on `stream`
 *    (a hipStream_t passed as void*; NULL = the default stream) and runs asynchronously.
 *  - Arguments are validated on the host before anything is enqueued; on any error nothing is
 *    enqueued and a negative frnn_status is returned.
 *  - The workspace is caller-owned device memory of at least the size the matching
 *    *_workspace_bytes function reports; its size does not depend on T for frnn_fwd. One
 *    workspace must not be used by two calls that may run concurrently.
 *  - Errors that can only be seen on the device (a bounded wait that ran out, a workgroup that
 *    landed on an unexpected accelerator die) are written into the workspace and reported by
 *    frnn_check() after the stream has reached the call.
 *  - Tensors are row-major with the layouts stated below, and 16-byte aligned. frnn_desc may give
 *    element strides for Wx, states and R (a time-major Wx, a [D, G*D] weight read in place);
 *    the other tensors are dense.
 */
#ifndef FRNN_H
#define FRNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FRNN_ABI_VERSION 2

/* Status codes (0 = success). */
enum {
  FRNN_OK = 0,
  FRNN_EINVAL = -1,          /* bad dimension, NULL required pointer, misaligned pointer, bad enum */
  FRNN_EUNSUPPORTED = -2,    /* valid request this build has no kernel for (dtype, D, path) */
  FRNN_EWORKSPACE = -3,      /* workspace NULL or smaller than required */
  FRNN_ENORESIDENT = -4,     /* the persistent grid cannot be co-resident on this device */
  FRNN_EHIP = -5,            /* a HIP runtime call failed */
  FRNN_ETIMEOUT = -6,        /* (frnn_check) a bounded inter-workgroup wait ran out */
  FRNN_EPLACEMENT = -7,      /* (frnn_check) a workgroup ran on another die than planned */
  FRNN_ENODEVICE = -8,       /* no usable gfx950 device */
  FRNN_ENOINIT = -9          /* frnn_init() has not prepared the current device */
};

/* Cells (FlashRNN cell names "lstm", "elman" and "gru"). */
enum { FRNN_CELL_LSTM = 0, FRNN_CELL_ELMAN = 1, FRNN_CELL_GRU = 2 };

/* Element types. */
enum { FRNN_F32 = 0, FRNN_BF16 = 1 };

/* Kernel designs (the FlashRNN page's "alternating" and "fused" variants, re-designed for
 * gfx950):
 *  ALTERNATING: per step one launch on `stream`: an MFMA kernel computes h.R for every head,
 *               R read from memory, and applies the gates in its epilogue (T launches); any
 *               head size runs.
 *  FUSED:       one persistent launch for all T steps (per chunk of batch rows where the batch
 *               exceeds one launch); R stays in registers (a quarter of it in LDS for LSTM
 *               and GRU heads of 1024 units, too wide for a die's registers). The workgroups
 *               sharing a head, all resident on one die, exchange h through that die's L2 every
 *               step; a head small enough for one workgroup keeps h in LDS. */
enum { FRNN_PATH_ALTERNATING = 0, FRNN_PATH_FUSED = 1 };

/* Problem description for frnn_fwd and frnn_bwd. G and S follow from `cell` (LSTM: 4, 2;
 * Elman: 1, 1; GRU: 3, 1).
 *
 * Strides are counted in elements of the tensor's own dtype; 0 selects the dense default given in
 * brackets. Inside a (batch row, step) slice Wx stays dense as [G, N, D] and states as [N, D]; in R
 * the unit axis e is contiguous. The FlashRNN usage example's layouts are the defaults; a strided
 * Wx lets a caller pass a time-major projection [T, B, G*N*D] (wx_sb = G*N*D, wx_st = B*G*N*D)
 * and a strided R the "5.3 LSTM" page's recurrent weight Wh [D, 4D] in place (N = 1, r_sg = D,
 * r_sd = 4D). Wx and states strides may be negative (a time- or batch-reversed view, the pointer
 * then addressing element [0, 0, ...]); their magnitudes must be multiples of 4. R strides must be
 * non-negative. Output views must not overlap themselves. frnn_bwd reads dstates with the states
 * strides, writes dWx with the Wx strides and dR with the R strides. */
typedef struct frnn_desc {
  int32_t B;          /* batch size, >= 1 */
  int32_t T;          /* sequence length, >= 0 */
  int32_t N;          /* number of heads, >= 1 */
  int32_t D;          /* head dimension, >= 1 (this build: a multiple of 32, <= 1024) */
  int32_t cell;       /* FRNN_CELL_* */
  int32_t in_dtype;   /* dtype of Wx, R, b, states0: FRNN_F32 or FRNN_BF16 */
  int32_t out_dtype;  /* dtype of states and last_states: FRNN_F32 (the only one supported) */
  int32_t reserved;   /* must be 0 */
  int64_t wx_sb;      /* Wx between batch rows             [T*G*N*D] */
  int64_t wx_st;      /* Wx between steps                  [G*N*D]   */
  int64_t st_ss;      /* states between h and c (LSTM)     [B*T*N*D] */
  int64_t st_sb;      /* states between batch rows         [T*N*D]   */
  int64_t st_st;      /* states between steps              [N*D]     */
  int64_t r_sg;       /* R between gates                   [N*D*D]   */
  int64_t r_sn;       /* R between heads                   [D*D]     */
  int64_t r_sd;       /* R between rows d (the input unit) [D]       */
} frnn_desc;

/* ABI version of the loaded library (FRNN_ABI_VERSION). */
int frnn_abi_version(void);

/* Prepares the current HIP device: checks that it is a gfx950 part, learns how the hardware deals
 * workgroups to accelerator dies (one probe kernel on a 1 KB buffer it allocates and frees, then a
 * device synchronisation) and raises the LDS limit of the persistent kernels. Call it once per
 * device before the first compute call on that device, outside stream capture; later calls
 * return at once. Thread-safe. Returns FRNN_OK, FRNN_ENODEVICE or FRNN_EHIP. */
int frnn_init(void);

/* Static, human-readable text for a status code. */
const char* frnn_status_str(int status);

/* Workspace bytes frnn_fwd needs for `d` on `path`. Returns FRNN_OK and writes *bytes, or a
 * negative status when `d` is invalid or unsupported. Independent of T. */
int frnn_workspace_bytes(const frnn_desc* d, int path, size_t* bytes);

/*
 * Head-wise forward recurrence (FlashRNN functional call: states, last_states = f(Wx, R, b,
 * states_initial)). Layouts (FlashRNN usage example):
 *   Wx          [B, T, G, N, D]   in_dtype, read-only (the already-projected input W.x)
 *   R           [G, N, D, D]      in_dtype, read-only; h (as a row vector) times R[g, n]
 *   b           [G, N, D]         in_dtype, read-only; NULL = zero bias
 *   states0     [S, B, 1, N, D]   in_dtype, read-only; NULL = zero initial h (and c)
 *   states      [S, B, T, N, D]   out_dtype, written; NULL = not written
 *   last_states [S, B, 1, N, D]   out_dtype, written; NULL = not written
 * For the LSTM, index 0 along S is h and index 1 is c. T == 0 is valid: last_states receives
 * states0 (or zeros) and states is untouched.
 */
int frnn_fwd(const frnn_desc* d, int path, const void* Wx, const void* R, const void* b,
             const void* states0, void* states, void* last_states, void* workspace,
             size_t workspace_bytes, void* stream);

/*
 * Backward of frnn_fwd (back-propagation through time). The FlashRNN usage example creates its
 * inputs with requires_grad; the pages print no gradient formulas, so this is the chain rule of
 * the cell equations above. For the loss
 *     L = sum(dstates * states) + sum(dlast * last_states)
 * it writes dWx = dL/dWx, dR = dL/dR, db = dL/db and dstates0 = dL/dstates0. Layouts:
 *   Wx, R, b, states0   as for frnn_fwd (in_dtype; b and states0 may be NULL = zeros)
 *   states      [S, B, T, N, D]   fp32, read-only: the states frnn_fwd returned for these inputs
 *                                 (required when T > 0; the backward recomputes the gates from them)
 *   dstates     [S, B, T, N, D]   fp32, read-only, or NULL = zeros
 *   dlast       [S, B, 1, N, D]   fp32, read-only, or NULL = zeros
 *   dWx         [B, T, G, N, D]   fp32, written, or NULL
 *   dR          [G, N, D, D]      fp32, written, or NULL
 *   db          [G, N, D]         fp32, written, or NULL
 *   dstates0    [S, B, 1, N, D]   fp32, written, or NULL
 * The contractions take bf16 operands (fp32 for fp32 inputs) with fp32 accumulation, like the
 * forward. T == 0: dstates0 = dlast, dR = db = 0. Both paths first recompute h.R for every step
 * with one MFMA GEMM (all heads in one launch) and end with one GEMM over all heads that forms dR
 * and db; they differ in the serial part, t = T-1 .. 0:
 *   FRNN_PATH_ALTERNATING: per step, one or two kernels (T or 2*T launches);
 *   FRNN_PATH_FUSED: one launch for all T steps (per chunk of batch rows where the batch
 *     exceeds one launch). Either one workgroup holds a whole head of 32 or 64 units and keeps
 *     that gradient in LDS, multiplying on the MFMA of the inputs' type (every head of at most
 *     64 units; on an Elman cell with the states in 16-byte aligned rows it reads h and dstates
 *     directly and the h.R recompute is skipped), or the workgroups of one die share a wider
 *     head and exchange the gradient reaching h through R every step (bf16 inputs; the
 *     forward's die-local design with h and R^T exchanged). LSTM and GRU heads of 1024 units
 *     keep part of R in LDS. Shapes this build has no fused design for (fp32 heads wider than 64
 *     units, say) return FRNN_EUNSUPPORTED before any launch; frnn_bwd_plan_str says which design
 *     a shape gets.
 * The workspace grows with T (it holds every step's h.R and gradient).
 */
int frnn_bwd(const frnn_desc* d, int path, const void* Wx, const void* R, const void* b,
             const void* states0, const void* states, const void* dstates, const void* dlast,
             void* dWx, void* dR, void* db, void* dstates0, void* workspace,
             size_t workspace_bytes, void* stream);

/* Workspace bytes frnn_bwd needs for `d` on `path` (grows with T). */
int frnn_bwd_workspace_bytes(const frnn_desc* d, int path, size_t* bytes);

/* Description of the launches frnn_bwd would make (for logs and tests). */
int frnn_bwd_plan_str(const frnn_desc* d, int path, char* buf, size_t cap);

/*
 * Plain multi-layer LSTM with input projection ("5.3 LSTM": MyLSTM.set_weights, MyLSTM.forward),
 * one direction or two (dirs = 1 or 2). Per layer l, direction k and step t:
 *   gates = in_t . Wi[l,k] + h . Wh[l,k] + (b_ih[l,k] + b_hh[l,k]),   column blocks i | f | g | o of width H
 *   c = f*c + i*g, h = o*tanh(c)
 * Direction 0 runs t = 0 .. T-1. Direction 1 (dirs = 2) is the same cell with its own weights run
 * over the sequence backwards, t = T-1 .. 0 (the page stores these "_reverse" weights; the reading
 * is torch.nn.LSTM's bidirectional layer). in_t = x[t] for l = 0, else layer l-1's output at step t,
 * the concatenation [h of direction 0, h of direction 1] at that step. Weights are indexed
 * [l * dirs + k]. Layouts (bf16 unless stated):
 *   x          [T, B, I]
 *   Wi[l,k]    [I, 4H] for l = 0, [dirs*H, 4H] for l >= 1   (host array of L*dirs device pointers)
 *   Wh[l,k]    [H, 4H]                                      (host array of L*dirs device pointers)
 *   b_ih[l,k], b_hh[l,k]  [4H]                              (host arrays; an entry may be NULL = 0)
 *   h0, c0     [L*dirs, B, H] or NULL (zeros)
 *   out        [T, B, dirs*H]  fp32, the top layer's output at every step (NULL = not written)
 *   hn, cn     [L*dirs, B, H]  fp32, final states (direction 1: after step t = 0) (NULL = not written)
 * The layers run in layer-major order (all T steps of layer 0, then layer 1), which gives the
 * same result as the page's time-major order because layer l at step t depends only on layer
 * l-1's outputs and on its own previous step. Each layer's projection over all T, both
 * directions at once, runs as one MFMA GEMM before its recurrence; the two directions' recurrences
 * run as two heads of one launch.
 */
int frnn_lstm_stack_fwd(int L, int dirs, int T, int B, int I, int H, int path, const void* x,
                        const void* const* Wi, const void* const* Wh, const void* const* b_ih,
                        const void* const* b_hh, const void* h0, const void* c0, void* out,
                        void* hn, void* cn, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Workspace bytes frnn_lstm_stack_fwd needs (grows with T: it holds the projected inputs). */
int frnn_lstm_stack_workspace_bytes(int L, int dirs, int T, int B, int I, int H, int path,
                                    size_t* bytes);

/*
 * Backward of frnn_lstm_stack_fwd, with one or two directions per layer (dirs as there; reading
 * of two directions: torch.nn.LSTM(bidirectional=True), whose state_dict "5.3 LSTM" reads): for
 * the loss
 *     L = sum(dout * out) + sum(dhn * hn) + sum(dcn * cn)
 * it writes the gradients of x, Wi[j], Wh[j], b_ih[j], b_hh[j], h0 and c0 ("5.3 LSTM"'s
 * parameters, j = l * dirs + k for layer l, direction k; the chain rule of its cell and
 * projection, the pages printing no gradients).
 * Inputs as for frnn_lstm_stack_fwd (bf16), plus (fp32, each may be NULL = zeros):
 *   dout [T, B, dirs*H],   dhn, dcn [L*dirs, B, H]
 * Outputs (fp32; a NULL pointer, or a NULL array, is not written):
 *   dx [T, B, I];  dWi[j] [in, 4H] (in = I for layer 0, else dirs*H);  dWh[j] [H, 4H];
 *   db_ih[j], db_hh[j] [4H] (equal: both biases enter as their sum);  dh0, dc0 [L*dirs, B, H]
 * The call runs the forward again, keeping every layer's projection and states in the workspace,
 * then per layer from the top and per direction: the head-wise backward (frnn_bwd's kernels on
 * `path`, with Wh read as R through strides, direction 1 through views that run from the last
 * step to the first), dWi = X^T . dWx, then dX = sum over directions of dWx . Wi^T (MFMA GEMMs,
 * bf16 operands, fp32 accumulation). T == 0: dh0 = dhn, dc0 = dcn, the weight gradients are zero.
 */
int frnn_lstm_stack_bwd(int L, int dirs, int T, int B, int I, int H, int path, const void* x,
                        const void* const* Wi, const void* const* Wh, const void* const* b_ih,
                        const void* const* b_hh, const void* h0, const void* c0, const void* dout,
                        const void* dhn, const void* dcn, void* dx, void* const* dWi,
                        void* const* dWh, void* const* db_ih, void* const* db_hh, void* dh0,
                        void* dc0, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes frnn_lstm_stack_bwd needs (grows with T and L). */
int frnn_lstm_stack_bwd_workspace_bytes(int L, int dirs, int T, int B, int I, int H, int path,
                                        size_t* bytes);

/* Waits for `stream`, then reads the device-side error word of the last call that used
 * `workspace` (FRNN_OK, FRNN_ETIMEOUT, FRNN_EPLACEMENT, or FRNN_EHIP if the wait failed).
 * workspace == NULL reads the word of frnn_fwd_noalloc's array on the current device. */
int frnn_check(const void* workspace, void* stream);

/* Bytes of the device array frnn_fwd_noalloc uses as its workspace (one per device). */
#define FRNN_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): frnn_fwd with the workspace replaced by a device array
 * the library holds, FRNN_NOALLOC_SCRATCH_BYTES per device, until the process ends (frnn_init()
 * looks its address up once per device). The call allocates nothing and frees nothing; it
 * returns FRNN_EWORKSPACE when the problem needs more than that (frnn_workspace_bytes says how
 * much) and FRNN_ENOINIT before frnn_init(). Every call on a device shares that device's array and
 * clears what it reads (the error word, the exchange words) at its start, so two calls that may
 * overlap on one device, on any streams, race and must not be made; frnn_check(NULL, stream)
 * reads the array's error word after the last call.
 */
int frnn_fwd_noalloc(const frnn_desc* d, int path, const void* Wx, const void* R, const void* b,
                     const void* states0, void* states, void* last_states, void* stream);

/* Description of the launch frnn_fwd would make for `d` on `path` (for logs and tests):
 * writes up to `cap` bytes of text into `buf`. Returns FRNN_OK or a negative status. */
int frnn_plan_str(const frnn_desc* d, int path, char* buf, size_t cap);

#ifdef __cplusplus
}
#endif

#endif /* FRNN_H */
