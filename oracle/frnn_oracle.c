/*
 * frnn_oracle.c -- plain, slow, fp64 CPU oracle for the head-wise LSTM / Elman / GRU forward
 * recurrence, its backward (back-propagation through time), and the plain multi-layer LSTM.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this file: it is
 * used by the test-suite, by the smoke check and by the benchmark's CPU-baseline leg. It shares no
 * code, header, table or constant with the HIP library.
 *
 * Sources of what is computed (cited by page title and section):
 *  - "FlashRNN: optimisation of RNNs on modern hardware" (hottg.com/neural/9889), usage example:
 *    tensor layouts Wx[B,T,G,N,D], R[G,N,D,D], b[G,N,D], states_initial[S,B,1,N,D],
 *    states[S,B,T,N,D]; for the LSTM the hidden state h is the first of [h, c]; the call returns
 *    (states, last_states). The page names the cells lstm / elman but prints no equations.
 *  - "5.3 LSTM" (developnotes.readthedocs.io, operator.html), MyLSTM.forward: per step
 *    ifgo = x_t*Wi + h*Wh + bias, split into four column blocks i, f, g, o; i, f, o pass a sigmoid,
 *    g a tanh; c = f*c + i*g; h = o*tanh(c); layer l >= 1 takes layer l-1's new h as its input;
 *    out[t] is the top layer's h; MyLSTM.set_weights: bias = bias_ih + bias_hh.
 *  - The head-wise reading: the 5.3 cell applied independently to every head n with that head's
 *    recurrent matrix R[:, n] (h as a row vector: pre[g][e] = sum_d h[d] * R[g,n,d,e]), the gate
 *    order along G being i, f, z (=g), o. Elman: h = tanh(Wx + h*R + b), G = 1, S = 1.
 *  - GRU (named in the FlashRNN page's list of cells, equations not printed): the textbook gated
 *    recurrent unit in the form where the reset gate scales the recurrent part of the candidate
 *    after its matrix product. G = 3 (r, z, n), S = 1. With a = h*R per gate:
 *      r = sigmoid(Wx_r + a_r + b_r),  z = sigmoid(Wx_z + a_z + b_z),
 *      n = tanh(Wx_n + r * (a_n + b_n)),  h_new = (1 - z) * n + z * h.
 *    Wx carries the input-side terms (the input projection and its biases); b holds the
 *    recurrent-side biases, b_n being the one inside the reset product.
 *
 * Everything is computed in double precision; inputs arrive already widened (exactly) to double.
 * Summation over d runs d = 0..D-1 in order for every output e. No blocking, fusion or reordering.
 * Batch rows and heads never interact, so (b, n) pairs run in parallel (OpenMP), which changes no
 * arithmetic.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_CELL_LSTM 0
#define ORACLE_CELL_ELMAN 1
#define ORACLE_CELL_GRU 2

/* Logistic sigmoid, textbook definition (5.3 LSTM: torch.sigmoid). */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

int oracle_abi_version(void) { return 1; }

/*
 * Head-wise forward (FlashRNN usage example layouts; 5.3 LSTM cell equations).
 *   Wx      [B,T,G,N,D]   already-projected inputs
 *   R       [G,N,D,D]     recurrent matrices, pre[g][e] += h[d] * R[g,n,d,e]
 *   b       [G,N,D]       bias, added every step
 *   states0 [S,B,1,N,D]   initial (h, c) or NULL for zeros
 *   states  [S,B,T,N,D]   state after consuming Wx[:,t] (NULL: not written)
 *   last    [S,B,1,N,D]   state after the last step (T == 0: the initial state); NULL: not written
 *   pairs   list of flattened (b*N + n) indices to compute, or NULL for all B*N
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_headwise_fwd(int cell, long B, long T, long N, long D, const double* Wx, const double* R,
                        const double* b, const double* states0, double* states, double* last,
                        const long* pairs, long npairs) {
  if (cell != ORACLE_CELL_LSTM && cell != ORACLE_CELL_ELMAN && cell != ORACLE_CELL_GRU) return -1;
  if (B <= 0 || N <= 0 || D <= 0 || T < 0) return -1;
  const long G = (cell == ORACLE_CELL_LSTM) ? 4 : (cell == ORACLE_CELL_GRU) ? 3 : 1;
  const long S = (cell == ORACLE_CELL_LSTM) ? 2 : 1;
  const long count = pairs ? npairs : B * N;
  int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (long p = 0; p < count; ++p) {
    const long bn = pairs ? pairs[p] : p;
    if (bn < 0 || bn >= B * N) { failed = 1; continue; }
    const long bi = bn / N, n = bn % N;
    double* h = (double*)malloc(sizeof(double) * D);
    double* c = (double*)malloc(sizeof(double) * D);
    double* hn = (double*)malloc(sizeof(double) * D);
    double* acc = (double*)malloc(sizeof(double) * G * D);
    double* pre = (double*)malloc(sizeof(double) * G * D);
    if (!h || !c || !hn || !acc || !pre) {
      failed = 1;
      free(h); free(c); free(hn); free(acc); free(pre);
      continue;
    }
    /* initial state: states0[s, bi, 0, n, :] or zeros */
    for (long e = 0; e < D; ++e) {
      h[e] = states0 ? states0[((0 * B + bi) * N + n) * D + e] : 0.0;
      c[e] = (S == 2 && states0) ? states0[((1 * B + bi) * N + n) * D + e] : 0.0;
    }
    for (long t = 0; t < T; ++t) {
      /* recurrent contraction with the previous step's full h (synchronous update) */
      for (long g = 0; g < G; ++g) {
        double* a = acc + g * D;
        for (long e = 0; e < D; ++e) a[e] = 0.0;
        for (long d = 0; d < D; ++d) {
          const double hd = h[d];
          const double* row = R + ((g * N + n) * D + d) * D;
          for (long e = 0; e < D; ++e) a[e] += hd * row[e];
        }
        /* pre-activation = Wx + R.h + b, in the order the equation is written (the GRU candidate
           keeps its recurrent part a_n + b_n apart: the reset gate scales it below) */
        for (long e = 0; e < D; ++e) {
          if (cell == ORACLE_CELL_GRU && g == 2) pre[g * D + e] = a[e] + b[(g * N + n) * D + e];
          else pre[g * D + e] = Wx[(((bi * T + t) * G + g) * N + n) * D + e] + a[e] + b[(g * N + n) * D + e];
        }
      }
      if (cell == ORACLE_CELL_LSTM) {
        for (long e = 0; e < D; ++e) {
          const double ig = sigmoid(pre[0 * D + e]);
          const double fg = sigmoid(pre[1 * D + e]);
          const double zg = tanh(pre[2 * D + e]);
          const double og = sigmoid(pre[3 * D + e]);
          c[e] = fg * c[e] + ig * zg;
          hn[e] = og * tanh(c[e]);
        }
      } else if (cell == ORACLE_CELL_GRU) {
        for (long e = 0; e < D; ++e) {
          const double rg = sigmoid(pre[0 * D + e]);
          const double zg = sigmoid(pre[1 * D + e]);
          const double ng = tanh(Wx[(((bi * T + t) * G + 2) * N + n) * D + e] + rg * pre[2 * D + e]);
          hn[e] = (1.0 - zg) * ng + zg * h[e];
        }
      } else {
        for (long e = 0; e < D; ++e) hn[e] = tanh(pre[e]);
      }
      memcpy(h, hn, sizeof(double) * D);
      if (states) {
        for (long e = 0; e < D; ++e) {
          states[(((0 * B + bi) * T + t) * N + n) * D + e] = h[e];
          if (S == 2) states[(((1 * B + bi) * T + t) * N + n) * D + e] = c[e];
        }
      }
    }
    if (last) {
      for (long e = 0; e < D; ++e) {
        last[((0 * B + bi) * N + n) * D + e] = h[e];
        if (S == 2) last[((1 * B + bi) * N + n) * D + e] = c[e];
      }
    }
    free(h); free(c); free(hn); free(acc); free(pre);
  }
  return failed ? -1 : 0;
}

/*
 * Head-wise backward (back-propagation through time) of oracle_headwise_fwd, for the loss
 *   L = sum(dstates * states) + sum(dlast * last_states),
 * i.e. given the gradients dstates [S,B,T,N,D] and dlast [S,B,1,N,D] of the two outputs (either
 * may be NULL for zeros) it returns
 *   dWx [B,T,G,N,D], dR [G,N,D,D], db [G,N,D], dstates0 [S,B,1,N,D]   (any may be NULL).
 * The pages print no gradient formulas; these are the chain rule applied to the forward cell
 * equations above (5.3 LSTM cell; Elman; the GRU reading), written out per step:
 *   LSTM: tc = tanh(c_t);  dc = dc_in + dh*o*(1 - tc^2);  d_o = dh*tc
 *         dpre_i = dc*z * i(1-i);  dpre_f = dc*c_{t-1} * f(1-f);  dpre_z = dc*i * (1-z^2);
 *         dpre_o = d_o * o(1-o);   dc carried to step t-1: dc*f
 *   Elman: dpre = dh * (1 - h_t^2)
 *   GRU:  dn = dh*(1-z);  dz = dh*(h_{t-1} - n);  dh carried directly to step t-1: dh*z
 *         dq = dn*(1-n^2) (q = the tanh argument);  dWx_n = dq;  da_n = dq*r;
 *         dr = dq*(a_n + b_n);  dpre_r = dr*r(1-r);  dpre_z = dz*z(1-z)
 * Here "da" is the gradient of the recurrent pre-activation part h*R (+ b): for the LSTM and
 * Elman da = dWx = dpre; for the GRU they differ in the n gate. Then
 *   dh_{t-1}[d] += sum_g sum_e da[g][e] * R[g,n,d,e]
 *   dR[g,n,d,e]  = sum_b sum_t h_{t-1}[b,n,d] * da_t[b][g][e],   db[g,n,e] = sum_b sum_t da_t[b][g][e]
 *   dstates0     = the gradient that reaches the initial state (h through R, plus the carried
 *                  direct parts: LSTM c, GRU h).
 * Each (b, n) row is run forward once more (keeping every step's gates and states), then walked
 * backwards from t = T-1 to 0. dR and db are summed afterwards in a fixed order (b, then t).
 */
int oracle_headwise_bwd(int cell, long B, long T, long N, long D, const double* Wx, const double* R,
                        const double* b, const double* states0, const double* dstates,
                        const double* dlast, double* dWx, double* dR, double* db, double* dstates0) {
  if (cell != ORACLE_CELL_LSTM && cell != ORACLE_CELL_ELMAN && cell != ORACLE_CELL_GRU) return -1;
  if (B <= 0 || N <= 0 || D <= 0 || T < 0) return -1;
  const long G = (cell == ORACLE_CELL_LSTM) ? 4 : (cell == ORACLE_CELL_GRU) ? 3 : 1;
  const long S = (cell == ORACLE_CELL_LSTM) ? 2 : 1;
  const long P = B * N;
  /* per (b, n) row: hh[t] = h before step t (hh[T] = after the last), cc likewise (LSTM),
     act[t][g][e] = gate values of step t, qn[t][e] = a_n + b_n (GRU), da[t][g][e] */
  double* hh = (double*)malloc(sizeof(double) * P * (T + 1) * D);
  double* cc = (double*)malloc(sizeof(double) * P * (T + 1) * D);
  double* act = (double*)malloc(sizeof(double) * P * (T > 0 ? T : 1) * G * D);
  double* qn = (double*)malloc(sizeof(double) * P * (T > 0 ? T : 1) * D);
  double* da = (double*)malloc(sizeof(double) * P * (T > 0 ? T : 1) * G * D);
  if (!hh || !cc || !act || !qn || !da) {
    free(hh); free(cc); free(act); free(qn); free(da);
    return -1;
  }
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long p = 0; p < P; ++p) {
    const long bi = p / N, n = p % N;
    double* H = hh + p * (T + 1) * D;
    double* C = cc + p * (T + 1) * D;
    double* A = act + p * (T > 0 ? T : 1) * G * D;
    double* Q = qn + p * (T > 0 ? T : 1) * D;
    double* DA = da + p * (T > 0 ? T : 1) * G * D;
    double* pre = (double*)malloc(sizeof(double) * G * D);
    double* dh = (double*)malloc(sizeof(double) * D);
    double* dc = (double*)malloc(sizeof(double) * D);
    double* dhn = (double*)malloc(sizeof(double) * D);
    if (!pre || !dh || !dc || !dhn) {
      free(pre); free(dh); free(dc); free(dhn);
#pragma omp atomic write
      failed = 1;
      continue;
    }
    for (long e = 0; e < D; ++e) {
      H[e] = states0 ? states0[((0 * B + bi) * N + n) * D + e] : 0.0;
      C[e] = (S == 2 && states0) ? states0[((1 * B + bi) * N + n) * D + e] : 0.0;
    }
    /* forward, keeping what the backward needs */
    for (long t = 0; t < T; ++t) {
      const double* h = H + t * D;
      for (long g = 0; g < G; ++g) {
        for (long e = 0; e < D; ++e) pre[g * D + e] = b[(g * N + n) * D + e];
        for (long d = 0; d < D; ++d) {
          const double* row = R + ((g * N + n) * D + d) * D;
          for (long e = 0; e < D; ++e) pre[g * D + e] += h[d] * row[e];
        }
      }
      double* a = A + t * G * D;
      for (long e = 0; e < D; ++e) {
        const double wx0 = Wx[(((bi * T + t) * G + 0) * N + n) * D + e];
        if (cell == ORACLE_CELL_LSTM) {
          const double ig = sigmoid(wx0 + pre[0 * D + e]);
          const double fg = sigmoid(Wx[(((bi * T + t) * G + 1) * N + n) * D + e] + pre[1 * D + e]);
          const double zg = tanh(Wx[(((bi * T + t) * G + 2) * N + n) * D + e] + pre[2 * D + e]);
          const double og = sigmoid(Wx[(((bi * T + t) * G + 3) * N + n) * D + e] + pre[3 * D + e]);
          a[0 * D + e] = ig; a[1 * D + e] = fg; a[2 * D + e] = zg; a[3 * D + e] = og;
          C[(t + 1) * D + e] = fg * C[t * D + e] + ig * zg;
          H[(t + 1) * D + e] = og * tanh(C[(t + 1) * D + e]);
        } else if (cell == ORACLE_CELL_GRU) {
          const double rg = sigmoid(wx0 + pre[0 * D + e]);
          const double zg = sigmoid(Wx[(((bi * T + t) * G + 1) * N + n) * D + e] + pre[1 * D + e]);
          const double ng = tanh(Wx[(((bi * T + t) * G + 2) * N + n) * D + e] + rg * pre[2 * D + e]);
          a[0 * D + e] = rg; a[1 * D + e] = zg; a[2 * D + e] = ng;
          Q[t * D + e] = pre[2 * D + e];
          H[(t + 1) * D + e] = (1.0 - zg) * ng + zg * h[e];
        } else {
          a[e] = tanh(wx0 + pre[e]);
          H[(t + 1) * D + e] = a[e];
        }
      }
    }
    /* backward: dh, dc hold the gradient reaching the state after step t */
    for (long e = 0; e < D; ++e) {
      dh[e] = dlast ? dlast[((0 * B + bi) * N + n) * D + e] : 0.0;
      dc[e] = (S == 2 && dlast) ? dlast[((1 * B + bi) * N + n) * D + e] : 0.0;
    }
    for (long t = T - 1; t >= 0; --t) {
      const double* a = A + t * G * D;
      double* dat = DA + t * G * D;
      for (long e = 0; e < D; ++e) {
        if (dstates) {
          dh[e] += dstates[(((0 * B + bi) * T + t) * N + n) * D + e];
          if (S == 2) dc[e] += dstates[(((1 * B + bi) * T + t) * N + n) * D + e];
        }
      }
      for (long e = 0; e < D; ++e) {
        double dw[4] = {0.0, 0.0, 0.0, 0.0};
        if (cell == ORACLE_CELL_LSTM) {
          const double ig = a[0 * D + e], fg = a[1 * D + e], zg = a[2 * D + e], og = a[3 * D + e];
          const double tc = tanh(C[(t + 1) * D + e]);
          const double dct = dc[e] + dh[e] * og * (1.0 - tc * tc);
          dw[0] = dct * zg * ig * (1.0 - ig);
          dw[1] = dct * C[t * D + e] * fg * (1.0 - fg);
          dw[2] = dct * ig * (1.0 - zg * zg);
          dw[3] = dh[e] * tc * og * (1.0 - og);
          for (long g = 0; g < 4; ++g) dat[g * D + e] = dw[g];
          dc[e] = dct * fg;
          dh[e] = 0.0; /* h_{t-1} is reached only through R, added below */
        } else if (cell == ORACLE_CELL_GRU) {
          const double rg = a[0 * D + e], zg = a[1 * D + e], ng = a[2 * D + e];
          const double dn = dh[e] * (1.0 - zg);
          const double dz = dh[e] * (H[t * D + e] - ng);
          const double dq = dn * (1.0 - ng * ng);
          dw[0] = dq * Q[t * D + e] * rg * (1.0 - rg);
          dw[1] = dz * zg * (1.0 - zg);
          dw[2] = dq;
          dat[0 * D + e] = dw[0];
          dat[1 * D + e] = dw[1];
          dat[2 * D + e] = dq * rg;
          dh[e] = dh[e] * zg; /* the direct part; the part through R is added below */
        } else {
          const double ht = a[e];
          dw[0] = dh[e] * (1.0 - ht * ht);
          dat[e] = dw[0];
          dh[e] = 0.0;
        }
        if (dWx)
          for (long g = 0; g < G; ++g) dWx[(((bi * T + t) * G + g) * N + n) * D + e] = dw[g];
      }
      /* gradient reaching h_{t-1} through the contraction */
      for (long d = 0; d < D; ++d) {
        double s = 0.0;
        for (long g = 0; g < G; ++g) {
          const double* row = R + ((g * N + n) * D + d) * D;
          for (long e = 0; e < D; ++e) s += dat[g * D + e] * row[e];
        }
        dhn[d] = s;
      }
      for (long d = 0; d < D; ++d) dh[d] += dhn[d];
    }
    if (dstates0) {
      for (long e = 0; e < D; ++e) {
        dstates0[((0 * B + bi) * N + n) * D + e] = dh[e];
        if (S == 2) dstates0[((1 * B + bi) * N + n) * D + e] = dc[e];
      }
    }
    free(pre); free(dh); free(dc); free(dhn);
  }
  if (!failed && (dR || db)) {
    /* dR[g,n,d,e] = sum_b sum_t h_{t-1}[d] da_t[g][e]; db[g,n,e] = sum_b sum_t da_t[g][e] */
#pragma omp parallel for schedule(dynamic, 1)
    for (long gn = 0; gn < G * N; ++gn) {
      const long g = gn / N, n = gn % N;
      for (long d = 0; d < D; ++d) {
        double* out = dR ? dR + ((g * N + n) * D + d) * D : NULL;
        if (out)
          for (long e = 0; e < D; ++e) out[e] = 0.0;
        for (long bi = 0; bi < B; ++bi) {
          const long p = bi * N + n;
          const double* H = hh + p * (T + 1) * D;
          const double* DA = da + p * (T > 0 ? T : 1) * G * D;
          for (long t = 0; t < T; ++t) {
            const double hd = H[t * D + d];
            if (out)
              for (long e = 0; e < D; ++e) out[e] += hd * DA[(t * G + g) * D + e];
          }
        }
      }
      if (db) {
        for (long e = 0; e < D; ++e) {
          double s = 0.0;
          for (long bi = 0; bi < B; ++bi) {
            const long p = bi * N + n;
            const double* DA = da + p * (T > 0 ? T : 1) * G * D;
            for (long t = 0; t < T; ++t) s += DA[(t * G + g) * D + e];
          }
          db[(g * N + n) * D + e] = s;
        }
      }
    }
  }
  free(hh); free(cc); free(act); free(qn); free(da);
  return failed ? -1 : 0;
}

/*
 * Plain multi-layer LSTM, 5.3 LSTM (MyLSTM.set_weights / MyLSTM.forward), unidirectional:
 *   x   [T,B,I] input sequence
 *   Wi[l] [in_l, 4H]  (in_0 = I, in_l = H for l >= 1); Wh[l] [H, 4H]
 *   b_ih[l], b_hh[l] [4H]; the bias used is their sum (set_weights)
 *   h0, c0 [L,B,H] or NULL for zeros
 *   out [T,B,H] top layer's h at every step; hn, cn [L,B,H] final states (NULL: not written)
 * The time loop is outermost and the layers run inside it, as the page writes it. Rows of the
 * batch are independent and run in parallel.
 */
int oracle_lstm_stack_p3(long L, long T, long B, long I, long H, const double* x,
                         const double* const* Wi, const double* const* Wh, const double* const* b_ih,
                         const double* const* b_hh, const double* h0, const double* c0, double* out,
                         double* hn, double* cn) {
  if (L <= 0 || B <= 0 || I <= 0 || H <= 0 || T < 0) return -1;
  const long H4 = 4 * H;
  int failed = 0;
  /* set_weights: bias = bias_ih + bias_hh */
  double* bias = (double*)malloc(sizeof(double) * L * H4);
  if (!bias) return -1;
  for (long l = 0; l < L; ++l)
    for (long j = 0; j < H4; ++j) bias[l * H4 + j] = b_ih[l][j] + b_hh[l][j];

#pragma omp parallel for schedule(dynamic, 1)
  for (long bi = 0; bi < B; ++bi) {
    double* h = (double*)malloc(sizeof(double) * L * H);
    double* c = (double*)malloc(sizeof(double) * L * H);
    double* xi = (double*)malloc(sizeof(double) * H4);
    double* hh = (double*)malloc(sizeof(double) * H4);
    double* ifgo = (double*)malloc(sizeof(double) * H4);
    if (!h || !c || !xi || !hh || !ifgo) {
      failed = 1;
      free(h); free(c); free(xi); free(hh); free(ifgo);
      continue;
    }
    for (long l = 0; l < L; ++l)
      for (long e = 0; e < H; ++e) {
        h[l * H + e] = h0 ? h0[(l * B + bi) * H + e] : 0.0;
        c[l * H + e] = c0 ? c0[(l * B + bi) * H + e] : 0.0;
      }
    for (long t = 0; t < T; ++t) {
      for (long l = 0; l < L; ++l) {
        /* layer input: x[t] for layer 0, the new h of layer l-1 otherwise */
        const double* in = (l == 0) ? x + (t * B + bi) * I : h + (l - 1) * H;
        const long K = (l == 0) ? I : H;
        for (long j = 0; j < H4; ++j) { xi[j] = 0.0; hh[j] = 0.0; }
        for (long k = 0; k < K; ++k) {
          const double v = in[k];
          const double* row = Wi[l] + k * H4;
          for (long j = 0; j < H4; ++j) xi[j] += v * row[j];
        }
        for (long k = 0; k < H; ++k) {
          const double v = h[l * H + k];
          const double* row = Wh[l] + k * H4;
          for (long j = 0; j < H4; ++j) hh[j] += v * row[j];
        }
        for (long j = 0; j < H4; ++j) ifgo[j] = xi[j] + hh[j] + bias[l * H4 + j];
        for (long e = 0; e < H; ++e) {
          const double ig = sigmoid(ifgo[0 * H + e]);
          const double fg = sigmoid(ifgo[1 * H + e]);
          const double gg = tanh(ifgo[2 * H + e]);
          const double og = sigmoid(ifgo[3 * H + e]);
          c[l * H + e] = fg * c[l * H + e] + ig * gg;
          h[l * H + e] = og * tanh(c[l * H + e]);
        }
      }
      if (out)
        for (long e = 0; e < H; ++e) out[(t * B + bi) * H + e] = h[(L - 1) * H + e];
    }
    for (long l = 0; l < L; ++l)
      for (long e = 0; e < H; ++e) {
        if (hn) hn[(l * B + bi) * H + e] = h[l * H + e];
        if (cn) cn[(l * B + bi) * H + e] = c[l * H + e];
      }
    free(h); free(c); free(xi); free(hh); free(ifgo);
  }
  free(bias);
  return failed ? -1 : 0;
}

/*
 * Multi-layer LSTM with one or two directions per layer. 5.3 LSTM (MyLSTM.__init__) takes a
 * `bidirectional` flag and set_weights copies the "_reverse" weights of each layer, but the page's
 * forward never uses them. The reading taken (the one of torch.nn.LSTM, whose state_dict names
 * the page copies): direction 1 of a layer is the same cell with its own weights, run over the
 * layer's input sequence from the last step to the first; the layer's output at step t is the
 * concatenation [h of direction 0 at t, h of direction 1 at t]; layer l >= 1 takes that
 * 2H-wide output as its input. With one direction this is the page's forward in layer-major
 * order.
 *   x   [T,B,I] input sequence
 *   Wi[j] [in_l, 4H] (in_0 = I, in_l = dirs*H), Wh[j] [H, 4H], b_ih[j], b_hh[j] [4H],
 *         for layer l and direction k at j = l*dirs + k; the bias used is b_ih + b_hh
 *   h0, c0 [L*dirs,B,H] or NULL for zeros
 *   out [T,B,dirs*H] the top layer's output at every step; hn, cn [L*dirs,B,H] the state each
 *       direction ends in (direction 1: after consuming step 0). NULL: not written.
 * Each layer runs whole before the next; each direction runs its own time loop. Batch rows are
 * independent and run in parallel.
 */
int oracle_lstm_stack_dirs(long L, long dirs, long T, long B, long I, long H, const double* x,
                           const double* const* Wi, const double* const* Wh, const double* const* b_ih,
                           const double* const* b_hh, const double* h0, const double* c0, double* out,
                           double* hn, double* cn) {
  if (L <= 0 || (dirs != 1 && dirs != 2) || B <= 0 || I <= 0 || H <= 0 || T < 0) return -1;
  const long H4 = 4 * H, W = dirs * H;  /* W: width of a layer's output */
  int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (long bi = 0; bi < B; ++bi) {
    double* prev = (double*)malloc(sizeof(double) * (T > 0 ? T : 1) * W);  /* layer input, l >= 1 */
    double* cur = (double*)malloc(sizeof(double) * (T > 0 ? T : 1) * W);   /* layer output */
    double* h = (double*)malloc(sizeof(double) * H);
    double* c = (double*)malloc(sizeof(double) * H);
    double* ifgo = (double*)malloc(sizeof(double) * H4);
    if (!prev || !cur || !h || !c || !ifgo) {
      failed = 1;
      free(prev); free(cur); free(h); free(c); free(ifgo);
      continue;
    }
    for (long l = 0; l < L; ++l) {
      const long K = (l == 0) ? I : W;
      for (long k = 0; k < dirs; ++k) {
        const long j = l * dirs + k;
        for (long e = 0; e < H; ++e) {
          h[e] = h0 ? h0[(j * B + bi) * H + e] : 0.0;
          c[e] = c0 ? c0[(j * B + bi) * H + e] : 0.0;
        }
        for (long s = 0; s < T; ++s) {
          const long t = (k == 0) ? s : T - 1 - s;  /* direction 1 walks the sequence backwards */
          const double* in = (l == 0) ? x + (t * B + bi) * I : prev + t * W;
          for (long q = 0; q < H4; ++q) ifgo[q] = b_ih[j][q] + b_hh[j][q];
          for (long d = 0; d < K; ++d) {
            const double v = in[d];
            const double* row = Wi[j] + d * H4;
            for (long q = 0; q < H4; ++q) ifgo[q] += v * row[q];
          }
          for (long d = 0; d < H; ++d) {
            const double v = h[d];
            const double* row = Wh[j] + d * H4;
            for (long q = 0; q < H4; ++q) ifgo[q] += v * row[q];
          }
          for (long e = 0; e < H; ++e) {
            const double ig = sigmoid(ifgo[0 * H + e]);
            const double fg = sigmoid(ifgo[1 * H + e]);
            const double gg = tanh(ifgo[2 * H + e]);
            const double og = sigmoid(ifgo[3 * H + e]);
            c[e] = fg * c[e] + ig * gg;
            h[e] = og * tanh(c[e]);
            cur[t * W + k * H + e] = h[e];
          }
        }
        for (long e = 0; e < H; ++e) {
          if (hn) hn[(j * B + bi) * H + e] = h[e];
          if (cn) cn[(j * B + bi) * H + e] = c[e];
        }
      }
      double* sw = prev; prev = cur; cur = sw;  /* this layer's output is the next one's input */
    }
    if (out)
      for (long t = 0; t < T; ++t)
        for (long q = 0; q < W; ++q) out[(t * B + bi) * W + q] = prev[t * W + q];
    free(prev); free(cur); free(h); free(c); free(ifgo);
  }
  return failed ? -1 : 0;
}
