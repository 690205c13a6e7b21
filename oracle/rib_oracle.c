/*
 * rib_oracle.c -- plain, slow, fp64 CPU oracle for RIB window attention with
 * the CLA output gate.  TEST INFRASTRUCTURE ONLY: the parity tests, the smoke
 * check and the benchmark's CPU-baseline leg call it; the GPU library never
 * links, loads or calls it, and it shares no code with that library.
 *
 * Method followed ("Rank-Factorized Implicit Neural Bias: Scaling
 * Super-Resolution Transformer with FlashAttention", as summarised on
 * gist.science (fr/it, "Methodologie proposee" / "Metodologia proposta",
 * part A) and on the omica.com.cn explainer, sections 2.2 and 2.3):
 *
 *   coordinate encoder   r = [c, sin(2^i c), cos(2^i c)]_{i<L},  c in [-1,1]^2
 *   implicit field       h = ReLU(r W_h + b_h),  Qp = h Wp_q,  Kp = h Wp_k
 *   attention            S = Qc Kc^T / sqrt(dh) + Qp Kp^T / sqrt(R)
 *   CLA gate             O = (softmax(S) V) * sigmoid(G)
 *
 * This file computes exactly that definition.  It does NOT use the channel
 * concatenation trick: the bias B = Qp Kp^T / sqrt(R) is materialised as its
 * own array (row by row) and added to the content score, then softmax, then
 * the V product, then the gate.  Everything is double precision; inputs are
 * the exact values of the caller's fp32 / bf16 tensors, upcast.
 *
 * Readings of points the pages leave open (each also listed in the design
 * notes of the repository):
 *   - coordinates include both endpoints, u(k) = -1 + 2k/(ws-1), and are
 *     float32 values (the pseudocode feeds a float tensor): the oracle rounds
 *     (2k-(ws-1))/(ws-1) to float once, then works in double;
 *   - coordinate order (y, x) with in-window index n = iy*ws + ix;
 *   - frequencies exactly 2^i, i = 0..L-1, no pi factor; the raw coordinates
 *     come first, then sin and cos for each frequency, y before x;
 *   - the hidden layer has a bias, the two rank heads have none;
 *   - one (Qp, Kp) pair shared by every head; D in 1/sqrt(D) is the head dim;
 *   - weights are stored W[in][out] row-major (y = x W);
 *   - maps that are not a multiple of the window: windows are anchored at
 *     (0,0), a window holds only the real tokens inside the map, and padded
 *     positions neither attend nor are attended to;
 *   - sigmoid(z) = 1 / (1 + exp(-z)), per element, G laid out like O.
 *
 * Packed weight layout (fp64 here, the same order the library takes in fp32):
 *   W_h[2+4L][hidden] | b_h[hidden] | Wp_q[hidden][R] | Wp_k[hidden][R]
 * Feature maps are NHWC: [B][H][W][heads*dh], head h owning channels
 * [h*dh, (h+1)*dh).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int rib_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* One coordinate value, as a float32, then widened: endpoints -1 and +1. */
static double coord_value(int k, int ws) {
  float num = (float)(2 * k - (ws - 1));
  float den = (float)(ws - 1);
  float u = num / den;
  return (double)u;
}

/* Fourier features of one token: out has 2 + 4L entries. */
static void fourier_features(double cy, double cx, int L, double* out) {
  int f = 0;
  out[f++] = cy;
  out[f++] = cx;
  for (int i = 0; i < L; ++i) {
    double freq = ldexp(1.0, i);
    out[f++] = sin(freq * cy);
    out[f++] = sin(freq * cx);
    out[f++] = cos(freq * cy);
    out[f++] = cos(freq * cx);
  }
}

/*
 * Encoder (explainer section 2.2, "coordinate encoding layer" and "implicit
 * neural field"): Qp, Kp are [ws*ws][R] row-major.  Returns 0, or -1 on a bad
 * argument.
 */
int rib_oracle_encode(int ws, int L, int hidden, int R, const double* weights,
                      double* qp, double* kp) {
  if (ws < 2 || L < 0 || hidden < 1 || R < 1 || !weights || !qp || !kp) return -1;
  const int F = 2 + 4 * L;
  const double* Wh = weights;
  const double* bh = Wh + (size_t)F * hidden;
  const double* Wq = bh + hidden;
  const double* Wk = Wq + (size_t)hidden * R;
  const int N = ws * ws;
  double* feat = (double*)malloc(sizeof(double) * F);
  double* h = (double*)malloc(sizeof(double) * hidden);
  if (!feat || !h) { free(feat); free(h); return -1; }
  for (int n = 0; n < N; ++n) {
    int iy = n / ws, ix = n % ws;
    fourier_features(coord_value(iy, ws), coord_value(ix, ws), L, feat);
    for (int j = 0; j < hidden; ++j) {
      double acc = bh[j];
      for (int f = 0; f < F; ++f) acc += feat[f] * Wh[(size_t)f * hidden + j];
      h[j] = acc > 0.0 ? acc : 0.0;
    }
    for (int r = 0; r < R; ++r) {
      double aq = 0.0, ak = 0.0;
      for (int j = 0; j < hidden; ++j) {
        aq += h[j] * Wq[(size_t)j * R + r];
        ak += h[j] * Wk[(size_t)j * R + r];
      }
      qp[(size_t)n * R + r] = aq;
      kp[(size_t)n * R + r] = ak;
    }
  }
  free(feat);
  free(h);
  return 0;
}

typedef struct {
  const double *qc, *kc, *v, *g, *qp, *kp;
  int B, H, W, heads, dh, R, ws;
  long tstride;  /* elements between the (Qp, Kp) tables of consecutive heads; 0 = one shared pair */
} problem;

static size_t elem(const problem* p, int b, int y, int x, int h, int d) {
  return (((size_t)b * p->H + y) * p->W + x) * (size_t)(p->heads * p->dh) + (size_t)h * p->dh + d;
}

/*
 * The real tokens of window (wy, wx): every map position whose window is
 * (floor(y/ws), floor(x/ws)) = (wy, wx), found by scanning the map.  Writes
 * their coordinates and in-window index n = (y mod ws)*ws + (x mod ws);
 * returns how many there are.
 */
static int window_tokens(const problem* p, int wy, int wx, int* ty, int* tx, int* tn) {
  int cnt = 0;
  for (int y = 0; y < p->H; ++y) {
    if (y / p->ws != wy) continue;
    for (int x = 0; x < p->W; ++x) {
      if (x / p->ws != wx) continue;
      ty[cnt] = y;
      tx[cnt] = x;
      tn[cnt] = (y % p->ws) * p->ws + (x % p->ws);
      ++cnt;
    }
  }
  return cnt;
}

/*
 * One query row i of one (image, window, head): content score row Sc, bias
 * row Bm, softmax row P, then O = (P V) * sigmoid(G) written to out (length
 * dh).  Sc, Bm, P are caller scratch of length nt.
 */
static void attend_row(const problem* p, int b, int h, int i, int nt, const int* ty, const int* tx,
                       const int* tn, double* Sc, double* Bm, double* P, double* out) {
  const double inv_sqrt_dh = 1.0 / sqrt((double)p->dh);
  const double inv_sqrt_r = 1.0 / sqrt((double)p->R);
  const double* q = p->qc + elem(p, b, ty[i], tx[i], h, 0);
  const double* qpos = p->qp + (size_t)h * p->tstride + (size_t)tn[i] * p->R;
  for (int j = 0; j < nt; ++j) {
    const double* k = p->kc + elem(p, b, ty[j], tx[j], h, 0);
    double s = 0.0;
    for (int d = 0; d < p->dh; ++d) s += q[d] * k[d];
    Sc[j] = s * inv_sqrt_dh;
    const double* kpos = p->kp + (size_t)h * p->tstride + (size_t)tn[j] * p->R;
    double bb = 0.0;
    for (int r = 0; r < p->R; ++r) bb += qpos[r] * kpos[r];
    Bm[j] = bb * inv_sqrt_r;
  }
  double mx = -INFINITY;
  for (int j = 0; j < nt; ++j) {
    double s = Sc[j] + Bm[j];
    P[j] = s;
    if (s > mx) mx = s;
  }
  double sum = 0.0;
  for (int j = 0; j < nt; ++j) {
    P[j] = exp(P[j] - mx);
    sum += P[j];
  }
  for (int j = 0; j < nt; ++j) P[j] /= sum;
  for (int d = 0; d < p->dh; ++d) {
    double a = 0.0;
    for (int j = 0; j < nt; ++j) a += P[j] * p->v[elem(p, b, ty[j], tx[j], h, d)];
    double gate = 1.0 / (1.0 + exp(-p->g[elem(p, b, ty[i], tx[i], h, d)]));
    out[d] = a * gate;
  }
}

static int check_problem(const problem* p) {
  if (!p->qc || !p->kc || !p->v || !p->g || !p->qp || !p->kp) return -1;
  if (p->B < 1 || p->H < 1 || p->W < 1 || p->heads < 1 || p->dh < 1 || p->R < 1 || p->ws < 2) return -1;
  return 0;
}

/*
 * Whole attention over a subset of (image, window, head) units.  Units are
 * numbered u = ((b*nWy + wy)*nWx + wx)*heads + h; the oracle computes units
 * [u_begin, u_end) and writes their outputs into o (full NHWC array; other
 * entries are left as they are).  u_end < 0 means all units.
 */
static int attn_units(const double* qc, const double* kc, const double* v, const double* g,
                      const double* qp, const double* kp, int B, int H, int W, int heads, int dh,
                      int R, int ws, long tstride, long u_begin, long u_end, double* o) {
  problem p = {qc, kc, v, g, qp, kp, B, H, W, heads, dh, R, ws, tstride};
  if (check_problem(&p) || !o) return -1;
  const int nWy = (H + ws - 1) / ws, nWx = (W + ws - 1) / ws;
  const long units = (long)B * nWy * nWx * heads;
  if (u_end < 0 || u_end > units) u_end = units;
  if (u_begin < 0) u_begin = 0;
  int fail = 0;
#pragma omp parallel
  {
    const int cap = ws * ws;
    int* ty = (int*)malloc(sizeof(int) * cap);
    int* tx = (int*)malloc(sizeof(int) * cap);
    int* tn = (int*)malloc(sizeof(int) * cap);
    double* Sc = (double*)malloc(sizeof(double) * cap);
    double* Bm = (double*)malloc(sizeof(double) * cap);
    double* P = (double*)malloc(sizeof(double) * cap);
    double* out = (double*)malloc(sizeof(double) * dh);
    if (!ty || !tx || !tn || !Sc || !Bm || !P || !out) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long u = u_begin; u < u_end; ++u) {
        int h = (int)(u % heads);
        long t = u / heads;
        int wx = (int)(t % nWx);
        t /= nWx;
        int wy = (int)(t % nWy);
        int b = (int)(t / nWy);
        int nt = window_tokens(&p, wy, wx, ty, tx, tn);
        for (int i = 0; i < nt; ++i) {
          attend_row(&p, b, h, i, nt, ty, tx, tn, Sc, Bm, P, out);
          for (int d = 0; d < dh; ++d) o[elem(&p, b, ty[i], tx[i], h, d)] = out[d];
        }
      }
    }
    free(ty); free(tx); free(tn); free(Sc); free(Bm); free(P); free(out);
  }
  return fail ? -1 : 0;
}

int rib_oracle_attn_units(const double* qc, const double* kc, const double* v, const double* g,
                          const double* qp, const double* kp, int B, int H, int W, int heads,
                          int dh, int R, int ws, long u_begin, long u_end, double* o) {
  return attn_units(qc, kc, v, g, qp, kp, B, H, W, heads, dh, R, ws, 0, u_begin, u_end, o);
}

/*
 * Per-head positional tables (the alternative to one shared pair): head h
 * uses Qp, Kp rows at qp + h*ws*ws*R, kp + h*ws*ws*R, i.e. tables laid out
 * [heads][ws*ws][R].  Everything else as rib_oracle_attn_units.
 */
int rib_oracle_attn_units_heads(const double* qc, const double* kc, const double* v, const double* g,
                                const double* qp, const double* kp, int B, int H, int W, int heads,
                                int dh, int R, int ws, long u_begin, long u_end, double* o) {
  return attn_units(qc, kc, v, g, qp, kp, B, H, W, heads, dh, R, ws, (long)ws * ws * R, u_begin, u_end, o);
}

int rib_oracle_attn(const double* qc, const double* kc, const double* v, const double* g,
                    const double* qp, const double* kp, int B, int H, int W, int heads, int dh,
                    int R, int ws, double* o) {
  return rib_oracle_attn_units(qc, kc, v, g, qp, kp, B, H, W, heads, dh, R, ws, 0, -1, o);
}

/*
 * Output rows for selected query tokens only (all heads): for each k < nq,
 * token (qb[k], qy[k], qx[k]) gets out[k][heads*dh].  Used to check full-size
 * problems at sampled positions.
 */
int rib_oracle_attn_rows(const double* qc, const double* kc, const double* v, const double* g,
                         const double* qp, const double* kp, int B, int H, int W, int heads,
                         int dh, int R, int ws, int nq, const int* qb, const int* qy,
                         const int* qx, double* out) {
  problem p = {qc, kc, v, g, qp, kp, B, H, W, heads, dh, R, ws, 0};
  if (check_problem(&p) || nq < 0 || (nq > 0 && (!qb || !qy || !qx || !out))) return -1;
  for (int k = 0; k < nq; ++k)
    if (qb[k] < 0 || qb[k] >= B || qy[k] < 0 || qy[k] >= H || qx[k] < 0 || qx[k] >= W) return -1;
  int fail = 0;
#pragma omp parallel
  {
    const int cap = ws * ws;
    int* ty = (int*)malloc(sizeof(int) * cap);
    int* tx = (int*)malloc(sizeof(int) * cap);
    int* tn = (int*)malloc(sizeof(int) * cap);
    double* Sc = (double*)malloc(sizeof(double) * cap);
    double* Bm = (double*)malloc(sizeof(double) * cap);
    double* P = (double*)malloc(sizeof(double) * cap);
    if (!ty || !tx || !tn || !Sc || !Bm || !P) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long t = 0; t < (long)nq * heads; ++t) {
        int k = (int)(t / heads), h = (int)(t % heads);
        int nt = window_tokens(&p, qy[k] / ws, qx[k] / ws, ty, tx, tn);
        int i = -1;
        for (int j = 0; j < nt; ++j)
          if (ty[j] == qy[k] && tx[j] == qx[k]) i = j;
        attend_row(&p, qb[k], h, i, nt, ty, tx, tn, Sc, Bm, P, out + ((size_t)k * heads + h) * dh);
      }
    }
    free(ty); free(tx); free(tn); free(Sc); free(Bm); free(P);
  }
  return fail ? -1 : 0;
}

/*
 * Row log-sum-exp of the scores (the normaliser of the softmax above):
 * lse[b][y][x][h] = log sum_j exp(Sc_ij + Bm_ij) over the real keys j of the
 * token's window.  This is what a training forward keeps for the backward
 * (explainer section 4.1 trains with the same attention).  One shared pair.
 */
static int attn_lse(const double* qc, const double* kc, const double* qp, const double* kp, int B, int H, int W,
                    int heads, int dh, int R, int ws, long tstride, double* lse) {
  problem p = {qc, kc, qc, qc, qp, kp, B, H, W, heads, dh, R, ws, tstride};
  if (check_problem(&p) || !lse) return -1;
  const int nWy = (H + ws - 1) / ws, nWx = (W + ws - 1) / ws;
  const long units = (long)B * nWy * nWx * heads;
  const double inv_sqrt_dh = 1.0 / sqrt((double)dh);
  const double inv_sqrt_r = 1.0 / sqrt((double)R);
  int fail = 0;
#pragma omp parallel
  {
    const int cap = ws * ws;
    int* ty = (int*)malloc(sizeof(int) * cap);
    int* tx = (int*)malloc(sizeof(int) * cap);
    int* tn = (int*)malloc(sizeof(int) * cap);
    double* S = (double*)malloc(sizeof(double) * cap);
    if (!ty || !tx || !tn || !S) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long u = 0; u < units; ++u) {
        int h = (int)(u % heads);
        long t = u / heads;
        int wx = (int)(t % nWx);
        t /= nWx;
        int wy = (int)(t % nWy);
        int b = (int)(t / nWy);
        int nt = window_tokens(&p, wy, wx, ty, tx, tn);
        for (int i = 0; i < nt; ++i) {
          const double* q = qc + elem(&p, b, ty[i], tx[i], h, 0);
          const double* qpos = qp + h * tstride + (size_t)tn[i] * R;
          double mx = -INFINITY;
          for (int j = 0; j < nt; ++j) {
            const double* k = kc + elem(&p, b, ty[j], tx[j], h, 0);
            const double* kpos = kp + h * tstride + (size_t)tn[j] * R;
            double sc = 0.0, bb = 0.0;
            for (int d = 0; d < dh; ++d) sc += q[d] * k[d];
            for (int r = 0; r < R; ++r) bb += qpos[r] * kpos[r];
            S[j] = sc * inv_sqrt_dh + bb * inv_sqrt_r;
            if (S[j] > mx) mx = S[j];
          }
          double sum = 0.0;
          for (int j = 0; j < nt; ++j) sum += exp(S[j] - mx);
          lse[(((size_t)b * H + ty[i]) * W + tx[i]) * heads + h] = mx + log(sum);
        }
      }
    }
    free(ty); free(tx); free(tn); free(S);
  }
  return fail ? -1 : 0;
}

int rib_oracle_attn_lse(const double* qc, const double* kc, const double* qp, const double* kp, int B, int H,
                        int W, int heads, int dh, int R, int ws, double* lse) {
  return attn_lse(qc, kc, qp, kp, B, H, W, heads, dh, R, ws, 0, lse);
}

/* The same with one (Qp, Kp) pair per head: qp, kp are [heads][ws*ws][R]. */
int rib_oracle_attn_lse_heads(const double* qc, const double* kc, const double* qp, const double* kp, int B,
                              int H, int W, int heads, int dh, int R, int ws, double* lse) {
  return attn_lse(qc, kc, qp, kp, B, H, W, heads, dh, R, ws, (long)ws * ws * R, lse);
}

/*
 * Debug view of one (image b, window (wy,wx), head h): the content score
 * matrix Sc, the explicit bias matrix Bm and the softmax P, each nt x nt
 * row-major over the window's real tokens in map scan order; token (y, x)
 * and in-window index n are returned in ty/tx/tn.  Caller provides arrays of
 * ws*ws entries (ws^4 for the matrices).  Returns nt, or -1.
 */
int rib_oracle_window_debug(const double* qc, const double* kc, const double* v, const double* g,
                            const double* qp, const double* kp, int B, int H, int W, int heads,
                            int dh, int R, int ws, int b, int wy, int wx, int h, double* Sc,
                            double* Bm, double* P, int* ty, int* tx, int* tn) {
  problem p = {qc, kc, v, g, qp, kp, B, H, W, heads, dh, R, ws, 0};
  if (check_problem(&p) || b < 0 || b >= B || h < 0 || h >= heads) return -1;
  int nt = window_tokens(&p, wy, wx, ty, tx, tn);
  double* out = (double*)malloc(sizeof(double) * dh);
  if (!out) return -1;
  for (int i = 0; i < nt; ++i)
    attend_row(&p, b, h, i, nt, ty, tx, tn, Sc + (size_t)i * nt, Bm + (size_t)i * nt,
               P + (size_t)i * nt, out);
  free(out);
  return nt;
}

/*
 * CLA gate producer (explainer section 2.3, the convolution path of CLA;
 * gist.science summaries part B: a depth-wise 3x3 convolution followed by a
 * point-wise 1x1 convolution produces the gating map):
 *
 *   D[b,y,x,c] = dw_b[c] + sum_{dy,dx in {-1,0,1}} X[b,y+dy,x+dx,c] * dw_w[c][dy+1][dx+1]
 *                (positions outside the map contribute zero: "same" padding, stride 1)
 *   G[b,y,x,o] = pw_b[o] + sum_c D[b,y,x,c] * pw_w[c][o]
 *
 * X and G are NHWC [B][H][W][C]; dw_w is [C][3][3], pw_w is [C_in][C_out]
 * (y = x W, the orientation used for every weight here).  D is kept per
 * token in double and never rounded.
 */
int rib_oracle_cla_gate(const double* x, const double* dw_w, const double* dw_b, const double* pw_w,
                        const double* pw_b, int B, int H, int W, int C, double* g) {
  if (B < 1 || H < 1 || W < 1 || C < 1) return -1;
  int fail = 0;
#pragma omp parallel
  {
    double* d = (double*)malloc(sizeof(double) * C);
    if (!d) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(static)
      for (long t = 0; t < (long)B * H * W; ++t) {
        int b = (int)(t / ((long)H * W)), y = (int)(t / W % H), xx = (int)(t % W);
        for (int c = 0; c < C; ++c) {
          double acc = dw_b[c];
          for (int dy = -1; dy <= 1; ++dy)
            for (int dx = -1; dx <= 1; ++dx) {
              int yy = y + dy, xs = xx + dx;
              if (yy < 0 || yy >= H || xs < 0 || xs >= W) continue;
              acc += x[(((size_t)b * H + yy) * W + xs) * C + c] * dw_w[(size_t)c * 9 + (dy + 1) * 3 + (dx + 1)];
            }
          d[c] = acc;
        }
        double* out = g + (size_t)t * C;
        for (int o = 0; o < C; ++o) {
          double acc = pw_b[o];
          for (int c = 0; c < C; ++c) acc += d[c] * pw_w[(size_t)c * C + o];
          out[o] = acc;
        }
      }
      free(d);
    }
  }
  return fail ? -1 : 0;
}

/*
 * Backward of RIB window attention with the gate (the training path the
 * pages time: explainer section 4.1, training time per iteration; the
 * forward as above).  Given dO, the gradient of a loss with respect to O,
 * per (image, window, head) and real tokens i, j of the window:
 *   s_ij  = qc_i.kc_j / sqrt(dh) + qp[n_i].kp[n_j] / sqrt(R),  P = softmax over j
 *   A_i   = sum_j P_ij v_j,   sg_i = sigmoid(g_i),   O_i = A_i * sg_i
 *   dA_i  = dO_i * sg_i
 *   dg_i  = dO_i * A_i * sg_i * (1 - sg_i)
 *   dP_ij = dA_i . v_j,   D_i = sum_j P_ij dP_ij,   dS_ij = P_ij (dP_ij - D_i)
 *   dqc_i = sum_j dS_ij kc_j / sqrt(dh),   dkc_j = sum_i dS_ij qc_i / sqrt(dh)
 *   dv_j  = sum_i P_ij dA_i
 *   dqp[n] = sum over every (image, window, head, i) with n_i = n of sum_j dS_ij kp[n_j] / sqrt(R)
 *   dkp[n] = sum over every (image, window, head, j) with n_j = n of sum_i dS_ij qp[n_i] / sqrt(R)
 * Row by row: each row of P, dP and dS is built in full before it is used.
 * dqp and dkp ([ws*ws][R]) are overwritten.
 */
static int attn_backward_unit(const problem* p, const double* dout, int b, int h, int nt, const int* ty,
                              const int* tx, const int* tn, double* prow, double* dprow, double* akv,
                              double* dkc_acc, double* dv_acc, double* dkp_acc, double* dqp_acc,
                              double* dqc, double* dkc, double* dv, double* dg) {
  const int dh = p->dh, R = p->R;
  const double inv_sqrt_dh = 1.0 / sqrt((double)dh);
  const double inv_sqrt_r = 1.0 / sqrt((double)R);
  memset(dkc_acc, 0, sizeof(double) * (size_t)nt * dh);
  memset(dv_acc, 0, sizeof(double) * (size_t)nt * dh);
  const double* qtab = p->qp + h * p->tstride;  /* this head's pair (the shared one when tstride = 0) */
  const double* ktab = p->kp + h * p->tstride;
  for (int i = 0; i < nt; ++i) {
    const double* q = p->qc + elem(p, b, ty[i], tx[i], h, 0);
    const double* qpos = qtab + (size_t)tn[i] * R;
    /* P row */
    double mx = -INFINITY;
    for (int j = 0; j < nt; ++j) {
      const double* k = p->kc + elem(p, b, ty[j], tx[j], h, 0);
      const double* kpos = ktab + (size_t)tn[j] * R;
      double sc = 0.0, bb = 0.0;
      for (int d = 0; d < dh; ++d) sc += q[d] * k[d];
      for (int r = 0; r < R; ++r) bb += qpos[r] * kpos[r];
      prow[j] = sc * inv_sqrt_dh + bb * inv_sqrt_r;
      if (prow[j] > mx) mx = prow[j];
    }
    double sum = 0.0;
    for (int j = 0; j < nt; ++j) {
      prow[j] = exp(prow[j] - mx);
      sum += prow[j];
    }
    for (int j = 0; j < nt; ++j) prow[j] /= sum;
    /* A_i, gate, dA_i, dg_i */
    double* dA = akv;  /* length dh */
    for (int d = 0; d < dh; ++d) {
      double a = 0.0;
      for (int j = 0; j < nt; ++j) a += prow[j] * p->v[elem(p, b, ty[j], tx[j], h, d)];
      const size_t e = elem(p, b, ty[i], tx[i], h, d);
      const double sg = 1.0 / (1.0 + exp(-p->g[e]));
      dA[d] = dout[e] * sg;
      dg[e] = dout[e] * a * sg * (1.0 - sg);
    }
    /* dP row, D_i */
    double D = 0.0;
    for (int j = 0; j < nt; ++j) {
      const double* vj = p->v + elem(p, b, ty[j], tx[j], h, 0);
      double dp = 0.0;
      for (int d = 0; d < dh; ++d) dp += dA[d] * vj[d];
      dprow[j] = dp;
      D += prow[j] * dp;
    }
    /* dS row and its contractions */
    double* dqi = dqc + elem(p, b, ty[i], tx[i], h, 0);
    for (int d = 0; d < dh; ++d) dqi[d] = 0.0;
    for (int j = 0; j < nt; ++j) {
      const double ds = prow[j] * (dprow[j] - D);
      const double* k = p->kc + elem(p, b, ty[j], tx[j], h, 0);
      const double* kpos = ktab + (size_t)tn[j] * R;
      for (int d = 0; d < dh; ++d) {
        dqi[d] += ds * k[d] * inv_sqrt_dh;
        dkc_acc[(size_t)j * dh + d] += ds * q[d] * inv_sqrt_dh;
        dv_acc[(size_t)j * dh + d] += prow[j] * dA[d];
      }
      for (int r = 0; r < R; ++r) {
        dqp_acc[(size_t)tn[i] * R + r] += ds * kpos[r] * inv_sqrt_r;
        dkp_acc[(size_t)tn[j] * R + r] += ds * qpos[r] * inv_sqrt_r;
      }
    }
  }
  for (int j = 0; j < nt; ++j)
    for (int d = 0; d < dh; ++d) {
      dkc[elem(p, b, ty[j], tx[j], h, d)] = dkc_acc[(size_t)j * dh + d];
      dv[elem(p, b, ty[j], tx[j], h, d)] = dv_acc[(size_t)j * dh + d];
    }
  return 0;
}

/* per_head = 0: one shared (Qp, Kp) pair, dqp and dkp [ws*ws][R] summed over
 * heads too; per_head = 1: qp, kp, dqp, dkp are [heads][ws*ws][R] and head h's
 * table gradient sums over images and windows only. */
static int attn_backward(const double* qc, const double* kc, const double* v, const double* g,
                         const double* qp, const double* kp, const double* dout, int B, int H, int W,
                         int heads, int dh, int R, int ws, int per_head, double* dqc, double* dkc, double* dv,
                         double* dg, double* dqp, double* dkp) {
  const size_t N = (size_t)ws * ws;
  problem p = {qc, kc, v, g, qp, kp, B, H, W, heads, dh, R, ws, per_head ? (long)(N * R) : 0};
  if (check_problem(&p) || !dout || !dqc || !dkc || !dv || !dg || !dqp || !dkp) return -1;
  const int nWy = (H + ws - 1) / ws, nWx = (W + ws - 1) / ws;
  const long units = (long)B * nWy * nWx * heads;
  const size_t NT = N * (size_t)R * (per_head ? (size_t)heads : 1);  /* table gradient entries */
  memset(dqp, 0, sizeof(double) * NT);
  memset(dkp, 0, sizeof(double) * NT);
  int fail = 0;
#pragma omp parallel
  {
    const int cap = ws * ws;
    int* ty = (int*)malloc(sizeof(int) * cap);
    int* tx = (int*)malloc(sizeof(int) * cap);
    int* tn = (int*)malloc(sizeof(int) * cap);
    double* prow = (double*)malloc(sizeof(double) * cap);
    double* dprow = (double*)malloc(sizeof(double) * cap);
    double* akv = (double*)malloc(sizeof(double) * dh);
    double* dkc_acc = (double*)malloc(sizeof(double) * (size_t)cap * dh);
    double* dv_acc = (double*)malloc(sizeof(double) * (size_t)cap * dh);
    double* dqp_t = (double*)calloc(NT, sizeof(double));
    double* dkp_t = (double*)calloc(NT, sizeof(double));
    if (!ty || !tx || !tn || !prow || !dprow || !akv || !dkc_acc || !dv_acc || !dqp_t || !dkp_t) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long u = 0; u < units; ++u) {
        int h = (int)(u % heads);
        long t = u / heads;
        int wx = (int)(t % nWx);
        t /= nWx;
        int wy = (int)(t % nWy);
        int b = (int)(t / nWy);
        int nt = window_tokens(&p, wy, wx, ty, tx, tn);
        const size_t toff = per_head ? (size_t)h * N * R : 0;
        attn_backward_unit(&p, dout, b, h, nt, ty, tx, tn, prow, dprow, akv, dkc_acc, dv_acc, dkp_t + toff,
                           dqp_t + toff, dqc, dkc, dv, dg);
      }
#pragma omp critical
      {
        for (size_t k = 0; k < NT; ++k) {
          dqp[k] += dqp_t[k];
          dkp[k] += dkp_t[k];
        }
      }
    }
    free(ty); free(tx); free(tn); free(prow); free(dprow); free(akv); free(dkc_acc); free(dv_acc);
    free(dqp_t); free(dkp_t);
  }
  return fail ? -1 : 0;
}

int rib_oracle_attn_backward(const double* qc, const double* kc, const double* v, const double* g,
                             const double* qp, const double* kp, const double* dout, int B, int H, int W,
                             int heads, int dh, int R, int ws, double* dqc, double* dkc, double* dv,
                             double* dg, double* dqp, double* dkp) {
  return attn_backward(qc, kc, v, g, qp, kp, dout, B, H, W, heads, dh, R, ws, 0, dqc, dkc, dv, dg, dqp, dkp);
}

/* The backward with one (Qp, Kp) pair per head (the per-head reading of the
 * explainer's section 2.2 attention rewrite): qp, kp, dqp, dkp are
 * [heads][ws*ws][R]; dqp[h], dkp[h] sum over every image and window of head h. */
int rib_oracle_attn_backward_heads(const double* qc, const double* kc, const double* v, const double* g,
                                   const double* qp, const double* kp, const double* dout, int B, int H, int W,
                                   int heads, int dh, int R, int ws, double* dqc, double* dkc, double* dv,
                                   double* dg, double* dqp, double* dkp) {
  return attn_backward(qc, kc, v, g, qp, kp, dout, B, H, W, heads, dh, R, ws, 1, dqc, dkc, dv, dg, dqp, dkp);
}

/*
 * Backward of the coordinate encoder (explainer section 2.2): given dQp, dKp
 * ([ws*ws][R]), the gradient of the packed weights W_h | b_h | Wp_q | Wp_k:
 *   pre = r W_h + b_h,  h = ReLU(pre),  Qp = h Wp_q,  Kp = h Wp_k
 *   dWp_q = sum_n h_n (x) dQp_n,  dWp_k = sum_n h_n (x) dKp_n
 *   dh_n = dQp_n Wp_q^T + dKp_n Wp_k^T,  dpre_n = dh_n * [pre_n > 0]
 *   dW_h = sum_n r_n (x) dpre_n,  db_h = sum_n dpre_n
 * (the derivative of ReLU at exactly 0 is taken as 0).  dweights is overwritten.
 */
int rib_oracle_encode_backward(int ws, int L, int hidden, int R, const double* weights, const double* dqp,
                               const double* dkp, double* dweights) {
  if (ws < 2 || L < 0 || hidden < 1 || R < 1) return -1;
  const int F = 2 + 4 * L;
  const double* Wh = weights;
  const double* bh = Wh + (size_t)F * hidden;
  const double* Wq = bh + hidden;
  const double* Wk = Wq + (size_t)hidden * R;
  double* dWh = dweights;
  double* dbh = dWh + (size_t)F * hidden;
  double* dWq = dbh + hidden;
  double* dWk = dWq + (size_t)hidden * R;
  memset(dweights, 0, sizeof(double) * ((size_t)F * hidden + hidden + 2 * (size_t)hidden * R));
  double* feat = (double*)malloc(sizeof(double) * F);
  double* pre = (double*)malloc(sizeof(double) * hidden);
  if (!feat || !pre) {
    free(feat); free(pre);
    return -1;
  }
  for (int n = 0; n < ws * ws; ++n) {
    const int iy = n / ws, ix = n % ws;
    fourier_features(coord_value(iy, ws), coord_value(ix, ws), L, feat);
    for (int j = 0; j < hidden; ++j) {
      double acc = bh[j];
      for (int f = 0; f < F; ++f) acc += feat[f] * Wh[(size_t)f * hidden + j];
      pre[j] = acc;
    }
    const double* gq = dqp + (size_t)n * R;
    const double* gk = dkp + (size_t)n * R;
    for (int j = 0; j < hidden; ++j) {
      const double hj = pre[j] > 0.0 ? pre[j] : 0.0;
      double dhj = 0.0;
      for (int r = 0; r < R; ++r) {
        dWq[(size_t)j * R + r] += hj * gq[r];
        dWk[(size_t)j * R + r] += hj * gk[r];
        dhj += gq[r] * Wq[(size_t)j * R + r] + gk[r] * Wk[(size_t)j * R + r];
      }
      const double dpre = pre[j] > 0.0 ? dhj : 0.0;
      dbh[j] += dpre;
      for (int f = 0; f < F; ++f) dWh[(size_t)f * hidden + j] += feat[f] * dpre;
    }
  }
  free(feat);
  free(pre);
  return 0;
}

/*
 * The attention's input projection in an SST block (explainer section 3.1:
 * each block applies LayerNorm, then RIB attention): per token (b, y, x) with
 * channels x_c, c < C,
 *   mu = (1/C) sum_c x_c,  var = (1/C) sum_c (x_c - mu)^2        (biased variance)
 *   xn_c = (x_c - mu) / sqrt(var + eps) * gamma_c + beta_c
 *   [q | k | v]_o = bias_o + sum_c xn_c * w[c][o],  o < 3C       (y = x W)
 * q, k, v are NHWC [B][H][W][C]; xn (if not NULL) receives LN(X), the input
 * the gate producer reads.
 */
int rib_oracle_ln_qkv(const double* x, const double* gamma, const double* beta, const double* w,
                      const double* bias, int B, int H, int W, int C, double eps, double* q, double* k,
                      double* v, double* xn) {
  if (!x || !gamma || !beta || !w || !bias || !q || !k || !v || B < 1 || H < 1 || W < 1 || C < 1 || !(eps >= 0.0))
    return -1;
  const long ntok = (long)B * H * W;
  int fail = 0;
#pragma omp parallel
  {
    double* row = (double*)malloc(sizeof(double) * C);
    if (!row) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(static)
      for (long t = 0; t < ntok; ++t) {
        const double* xt = x + t * C;
        double mu = 0.0;
        for (int c = 0; c < C; ++c) mu += xt[c];
        mu /= C;
        double var = 0.0;
        for (int c = 0; c < C; ++c) var += (xt[c] - mu) * (xt[c] - mu);
        var /= C;
        const double inv = 1.0 / sqrt(var + eps);
        for (int c = 0; c < C; ++c) row[c] = (xt[c] - mu) * inv * gamma[c] + beta[c];
        if (xn)
          for (int c = 0; c < C; ++c) xn[t * C + c] = row[c];
        for (int o = 0; o < 3 * C; ++o) {
          double acc = bias[o];
          for (int c = 0; c < C; ++c) acc += row[c] * w[(size_t)c * 3 * C + o];
          double* dst = o < C ? q : (o < 2 * C ? k : v);
          dst[t * C + o % C] = acc;
        }
      }
    }
    free(row);
  }
  return fail ? -1 : 0;
}

/*
 * Space-time windows (explainer section 6: for video, the coordinate MLP takes
 * spatio-temporal coordinates and the attention windows become 3-D).
 * A video map is [B][T][H][W][C]; a window spans wt frames x ws rows x ws
 * columns, anchored at (0, 0, 0); in-window index n = (it*ws + iy)*ws + ix.
 */

/* temporal coordinate: the same float32 grid over wt points; 0 for a single frame */
static double coord_value_t(int k, int wt) { return wt == 1 ? 0.0 : coord_value(k, wt); }

/* [c_t, c_y, c_x], then for each frequency 2^i: sin t, sin y, sin x, cos t, cos y, cos x */
static void fourier_features3(double ct, double cy, double cx, int L, double* out) {
  int f = 0;
  out[f++] = ct;
  out[f++] = cy;
  out[f++] = cx;
  for (int i = 0; i < L; ++i) {
    const double freq = ldexp(1.0, i);
    out[f++] = sin(freq * ct);
    out[f++] = sin(freq * cy);
    out[f++] = sin(freq * cx);
    out[f++] = cos(freq * ct);
    out[f++] = cos(freq * cy);
    out[f++] = cos(freq * cx);
  }
}

/* Encoder over a wt x ws x ws window: Qp, Kp [wt*ws*ws][R]; weights W_h[(3+6L)][hidden] | b_h | Wp_q | Wp_k. */
int rib_oracle_encode3d(int wt, int ws, int L, int hidden, int R, const double* weights, double* qp, double* kp) {
  if (wt < 1 || ws < 2 || L < 0 || hidden < 1 || R < 1 || !weights || !qp || !kp) return -1;
  const int F = 3 + 6 * L;
  const double* Wh = weights;
  const double* bh = Wh + (size_t)F * hidden;
  const double* Wq = bh + hidden;
  const double* Wk = Wq + (size_t)hidden * R;
  double* feat = (double*)malloc(sizeof(double) * F);
  double* h = (double*)malloc(sizeof(double) * hidden);
  if (!feat || !h) {
    free(feat); free(h);
    return -1;
  }
  for (int it = 0; it < wt; ++it)
    for (int iy = 0; iy < ws; ++iy)
      for (int ix = 0; ix < ws; ++ix) {
        const int n = (it * ws + iy) * ws + ix;
        fourier_features3(coord_value_t(it, wt), coord_value(iy, ws), coord_value(ix, ws), L, feat);
        for (int j = 0; j < hidden; ++j) {
          double acc = bh[j];
          for (int f = 0; f < F; ++f) acc += feat[f] * Wh[(size_t)f * hidden + j];
          h[j] = acc > 0.0 ? acc : 0.0;
        }
        for (int r = 0; r < R; ++r) {
          double aq = 0.0, ak = 0.0;
          for (int j = 0; j < hidden; ++j) {
            aq += h[j] * Wq[(size_t)j * R + r];
            ak += h[j] * Wk[(size_t)j * R + r];
          }
          qp[(size_t)n * R + r] = aq;
          kp[(size_t)n * R + r] = ak;
        }
      }
  free(feat);
  free(h);
  return 0;
}

/*
 * Attention over space-time windows, the 2-D definition with 3-D windows: per
 * (image, window, head) and real query i, S = Qc Kc^T / sqrt(dh) + Qp[n_i] Kp[n_j]^T / sqrt(R)
 * over the window's real tokens j, softmax, times V, gated by sigmoid(G).
 * The window's tokens are found by scanning the whole video.
 */
int rib_oracle_attn3d(const double* qc, const double* kc, const double* v, const double* g, const double* qp,
                      const double* kp, int B, int T, int H, int W, int heads, int dh, int R, int wt, int ws,
                      double* o) {
  if (!qc || !kc || !v || !g || !qp || !kp || !o || B < 1 || T < 1 || H < 1 || W < 1 || heads < 1 || dh < 1 ||
      R < 1 || wt < 1 || ws < 2)
    return -1;
  const int C = heads * dh;
  const int nWt = (T + wt - 1) / wt, nWy = (H + ws - 1) / ws, nWx = (W + ws - 1) / ws;
  const long units = (long)B * nWt * nWy * nWx * heads;
  const double inv_sqrt_dh = 1.0 / sqrt((double)dh), inv_sqrt_r = 1.0 / sqrt((double)R);
  int fail = 0;
#pragma omp parallel
  {
    const int cap = wt * ws * ws;
    long* off = (long*)malloc(sizeof(long) * cap);
    int* tn = (int*)malloc(sizeof(int) * cap);
    double* P = (double*)malloc(sizeof(double) * cap);
    if (!off || !tn || !P) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long u = 0; u < units; ++u) {
        const int h = (int)(u % heads);
        long r = u / heads;
        const int wx = (int)(r % nWx);
        r /= nWx;
        const int wy = (int)(r % nWy);
        r /= nWy;
        const int wtw = (int)(r % nWt);
        const int b = (int)(r / nWt);
        int nt = 0;
        for (int t = 0; t < T; ++t) {
          if (t / wt != wtw) continue;
          for (int y = 0; y < H; ++y) {
            if (y / ws != wy) continue;
            for (int x = 0; x < W; ++x) {
              if (x / ws != wx) continue;
              off[nt] = ((((long)b * T + t) * H + y) * W + x) * C + (long)h * dh;
              tn[nt] = ((t % wt) * ws + y % ws) * ws + x % ws;
              ++nt;
            }
          }
        }
        for (int i = 0; i < nt; ++i) {
          double mx = -INFINITY;
          for (int j = 0; j < nt; ++j) {
            double sc = 0.0, bb = 0.0;
            for (int d = 0; d < dh; ++d) sc += qc[off[i] + d] * kc[off[j] + d];
            for (int k = 0; k < R; ++k) bb += qp[(size_t)tn[i] * R + k] * kp[(size_t)tn[j] * R + k];
            P[j] = sc * inv_sqrt_dh + bb * inv_sqrt_r;
            if (P[j] > mx) mx = P[j];
          }
          double sum = 0.0;
          for (int j = 0; j < nt; ++j) {
            P[j] = exp(P[j] - mx);
            sum += P[j];
          }
          for (int d = 0; d < dh; ++d) {
            double a = 0.0;
            for (int j = 0; j < nt; ++j) a += P[j] * v[off[j] + d];
            o[off[i] + d] = a / sum / (1.0 + exp(-g[off[i] + d]));
          }
        }
      }
    }
    free(off); free(tn); free(P);
  }
  return fail ? -1 : 0;
}
