/*
 * rnn_oracle.c -- plain, slow, double-precision CPU oracle for the ONNX
 * recurrent layers (RNN, GRU, LSTM).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or constant table with the
 * HIP library.
 *
 * What it follows ("Recurrent layers" page of the OneGpu docs, recursiveai.org):
 *   - introduction: cells, directions, layouts, options, the eleven activations
 *     with alpha/beta already resolved; weights used as stored, gate order
 *     i,o,f,c (LSTM) and z,r,h (GRU);
 *   - "Arithmetic and determinism": pre = ((xw + rec) + Wb) + Rb, then the
 *     peephole terms (i and f with the previous cell state, o with the new one),
 *     then clip, then the activation, then c = f*c + i*c~, h = o*h_act(c);
 *     GRU h = (1 - z)*h~ + z*h;
 *   - "Semantics": sequence_lens (reverse starts at len-1, Y zero past len,
 *     Y_h/Y_c the state after the last valid step, len 0 gives zero states,
 *     len above Seq acts as Seq), Seq = 0 gives the initial states, clip
 *     clamps every gate pre-activation when positive with NaN passing,
 *     input_forget f = 1 - i, linear_before_reset = 1 form;
 *   - tensor shapes and activation formulas of the ONNX operator definitions,
 *     which the page defers to.
 * Readings where the page is silent are listed in the design notes; the two
 * that touch this file are: the peephole term is added after the bias sum, and
 * the GRU candidate with linear_before_reset = 0 is
 * ((xw_h + R_h.(r*h)) + Wb_h) + Rb_h.
 *
 * Everything is evaluated in double precision, one (direction, batch row)
 * sequence at a time; the input projection is written as plain dot products
 * inside the step loop, not as a matrix product.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Cell and activation codes of this file (independent of any library enum). */
enum { OR_RNN = 0, OR_GRU = 1, OR_LSTM = 2 };
enum { OR_FORWARD = 0, OR_REVERSE = 1, OR_BIDIRECTIONAL = 2 };
enum {
  OR_RELU = 0, OR_TANH, OR_SIGMOID, OR_AFFINE, OR_LEAKYRELU, OR_THRESHOLDEDRELU,
  OR_SCALEDTANH, OR_HARDSIGMOID, OR_ELU, OR_SOFTSIGN, OR_SOFTPLUS
};

typedef struct {
  int cell;            /* OR_RNN / OR_GRU / OR_LSTM */
  int direction;       /* OR_FORWARD / OR_REVERSE / OR_BIDIRECTIONAL */
  int layout;          /* 0: X [S,B,I], Y [S,D,B,H]; 1: X [B,S,I], Y [B,S,D,H] */
  int64_t seq, batch, input, hidden;
  double clip;         /* applied when > 0 */
  int input_forget;    /* LSTM only */
  int linear_before_reset; /* GRU only */
  int64_t max_length;  /* 0: none; otherwise a bound on the steps run */
  int act_kind[6];     /* per direction: LSTM f,g,h; GRU f,g; RNN f */
  double act_alpha[6];
  double act_beta[6];
} oracle_problem;

/* ONNX activation functions (operator definitions), evaluated in double. */
double oracle_activation(int kind, double alpha, double beta, double x) {
  switch (kind) {
    case OR_RELU: return x < 0.0 ? 0.0 : x;              /* max(0, x); NaN passes */
    case OR_TANH: return tanh(x);
    case OR_SIGMOID: return 1.0 / (1.0 + exp(-x));
    case OR_AFFINE: return alpha * x + beta;
    case OR_LEAKYRELU: return x >= 0.0 ? x : alpha * x;
    case OR_THRESHOLDEDRELU: return x > alpha ? x : 0.0;
    case OR_SCALEDTANH: return alpha * tanh(beta * x);
    case OR_HARDSIGMOID: {
      double v = alpha * x + beta;
      if (v < 0.0) v = 0.0;
      if (v > 1.0) v = 1.0;
      return v;
    }
    case OR_ELU: return x >= 0.0 ? x : alpha * (exp(x) - 1.0);
    case OR_SOFTSIGN: return x / (1.0 + fabs(x));
    case OR_SOFTPLUS: return x > 700.0 ? x : log1p(exp(x)); /* log(1 + e^x) */
    default: return NAN;
  }
}

/* clip: clamp to [-clip, clip] when clip > 0; comparisons let NaN through. */
static double clipv(double x, double clip) {
  if (clip > 0.0) {
    if (x < -clip) return -clip;
    if (x > clip) return clip;
  }
  return x;
}

static int gates_of(int cell) { return cell == OR_LSTM ? 4 : (cell == OR_GRU ? 3 : 1); }
static int slots_of(int cell) { return cell == OR_LSTM ? 3 : (cell == OR_GRU ? 2 : 1); }

/* Plain matrix product C[m][n] = sum_k A[m][k] * Bt[n][k] (B given as its
 * transpose, N x K row-major).  Used only to check the library's projection. */
void oracle_projection(int64_t M, int64_t N, int64_t K, const double* A, const double* Bt, double* C) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) s += A[m * K + k] * Bt[n * K + k];
      C[m * N + n] = s;
    }
}

/* Bits of the IEEE binary16 value nearest to x, ties to even: how a Half
 * output holds a result ("How a layer runs", item 4: the outputs are rounded
 * to Half; "Tolerance and evidence": Half outputs rounded from float32
 * state).  Written from the format's definition: 1 sign bit, 5 exponent bits
 * (bias 15), 10 fraction bits; normal numbers in [2^-14, 65504], subnormals
 * multiples of 2^-24; a magnitude of 65520 (65504 plus half its spacing) or
 * more overflows to infinity.  rint rounds to nearest even in the default
 * rounding mode, and every division below is by a power of two, so exact. */
uint16_t oracle_round_half(double x) {
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  const double a = fabs(x);
  if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  if (a < ldexp(1.0, -14)) {                        /* subnormal (or zero): spacing 2^-24 */
    const double q = rint(a / ldexp(1.0, -24));     /* 0 .. 1024; 1024 is the smallest normal */
    return (uint16_t)(sign | (uint16_t)q);
  }
  int e2 = 0;
  (void)frexp(a, &e2);                              /* a = m * 2^e2, m in [0.5, 1) */
  int e = e2 - 1;                                   /* a in [2^e, 2^(e+1)) */
  double q = rint(a / ldexp(1.0, e - 10));          /* significand in units of the spacing: 1024 .. 2048 */
  if (q == 2048.0) {
    q = 1024.0;
    e += 1;
  }
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q - 1024.0));
}

static double dot(const double* a, const double* b, int64_t n) {
  double s = 0.0;
  for (int64_t k = 0; k < n; ++k) s += a[k] * b[k];
  return s;
}

/* One (direction d, batch row b) sequence. */
static void run_sequence(const oracle_problem* p, int64_t d, int64_t b,
                         const double* X, const double* W, const double* R, const double* Bias,
                         const int32_t* lens, const double* init_h, const double* init_c, const double* P,
                         double* Y, double* Y_h, double* Y_c, double* work) {
  const int64_t S = p->seq, B = p->batch, I = p->input, H = p->hidden;
  const int64_t D = p->direction == OR_BIDIRECTIONAL ? 2 : 1;
  const int G = gates_of(p->cell);
  const int reverse = (p->direction == OR_REVERSE) || (p->direction == OR_BIDIRECTIONAL && d == 1);
  const int ns = slots_of(p->cell);
  const int* ak = p->act_kind + d * ns;
  const double* aa = p->act_alpha + d * ns;
  const double* ab = p->act_beta + d * ns;

  const double* Wd = W + d * (int64_t)G * H * I;       /* [G*H, I] */
  const double* Rd = R + d * (int64_t)G * H * H;       /* [G*H, H] */
  const double* Wb = Bias ? Bias + d * 2 * (int64_t)G * H : NULL;
  const double* Rb = Bias ? Wb + (int64_t)G * H : NULL;
  const double* Pd = P ? P + d * 3 * H : NULL;        /* i, o, f */

  double* h = work;              /* H */
  double* c = h + H;             /* H */
  double* hn = c + H;            /* H */
  double* cn = hn + H;           /* H */
  double* xw = cn + H;           /* G*H */
  double* rec = xw + G * H;      /* G*H */
  double* rh = rec + G * H;      /* H: r * h for the GRU candidate */
  double* gz = rh + H;           /* H: GRU z */
  double* gr = gz + H;           /* H: GRU r */

  /* state index per layout: L0 [D,B,H], L1 [B,D,H] */
  const int64_t sidx = p->layout == 0 ? (d * B + b) * H : (b * D + d) * H;
  for (int64_t j = 0; j < H; ++j) {
    h[j] = init_h ? init_h[sidx + j] : 0.0;
    c[j] = init_c ? init_c[sidx + j] : 0.0;
  }

  if (S == 0) {                          /* nothing runs: initial states or zeros */
    if (Y_h) for (int64_t j = 0; j < H; ++j) Y_h[sidx + j] = h[j];
    if (Y_c) for (int64_t j = 0; j < H; ++j) Y_c[sidx + j] = c[j];
    return;
  }

  int64_t L = S;
  if (lens) {
    L = lens[b];
    if (L < 0) L = 0;
    if (L > S) L = S;
  }
  if (p->max_length > 0 && L > p->max_length) L = p->max_length;

  for (int64_t s = 0; s < L; ++s) {
    const int64_t t = reverse ? L - 1 - s : s;
    const double* x = X + (p->layout == 0 ? (t * B + b) * I : (b * S + t) * I);
    for (int64_t n = 0; n < G * H; ++n) {
      xw[n] = dot(Wd + n * I, x, I);
      rec[n] = dot(Rd + n * H, h, H);
    }
    if (p->cell == OR_LSTM) {
      /* gate blocks of W, R, Wb, Rb: i (0), o (1), f (2), c (3); P: i, o, f */
      for (int64_t j = 0; j < H; ++j) {
        double pre[4];
        for (int g = 0; g < 4; ++g) {
          const int64_t n = g * H + j;
          pre[g] = ((xw[n] + rec[n]) + (Wb ? Wb[n] : 0.0)) + (Rb ? Rb[n] : 0.0);
        }
        double pi = pre[0] + (Pd ? Pd[j] * c[j] : 0.0);
        double pf = pre[2] + (Pd ? Pd[2 * H + j] * c[j] : 0.0);
        double pc = pre[3];
        pi = clipv(pi, p->clip);
        pf = clipv(pf, p->clip);
        pc = clipv(pc, p->clip);
        const double ig = oracle_activation(ak[0], aa[0], ab[0], pi);
        const double fg = p->input_forget ? 1.0 - ig : oracle_activation(ak[0], aa[0], ab[0], pf);
        const double ct = oracle_activation(ak[1], aa[1], ab[1], pc);
        const double cnew = fg * c[j] + ig * ct;
        double po = pre[1] + (Pd ? Pd[H + j] * cnew : 0.0);
        po = clipv(po, p->clip);
        const double og = oracle_activation(ak[0], aa[0], ab[0], po);
        cn[j] = cnew;
        hn[j] = og * oracle_activation(ak[2], aa[2], ab[2], cnew);
      }
    } else if (p->cell == OR_GRU) {
      /* gate blocks: z (0), r (1), h (2) */
      for (int64_t j = 0; j < H; ++j) {
        const int64_t nz = j, nr = H + j;
        double pz = ((xw[nz] + rec[nz]) + (Wb ? Wb[nz] : 0.0)) + (Rb ? Rb[nz] : 0.0);
        double pr = ((xw[nr] + rec[nr]) + (Wb ? Wb[nr] : 0.0)) + (Rb ? Rb[nr] : 0.0);
        gz[j] = oracle_activation(ak[0], aa[0], ab[0], clipv(pz, p->clip));
        gr[j] = oracle_activation(ak[0], aa[0], ab[0], clipv(pr, p->clip));
      }
      for (int64_t k = 0; k < H; ++k) rh[k] = gr[k] * h[k];
      for (int64_t j = 0; j < H; ++j) {
        const int64_t nh = 2 * H + j;
        const double wbh = Wb ? Wb[nh] : 0.0, rbh = Rb ? Rb[nh] : 0.0;
        double ph;
        if (p->linear_before_reset) {
          ph = (xw[nh] + gr[j] * (rec[nh] + rbh)) + wbh;
        } else {
          const double rech = dot(Rd + nh * H, rh, H);   /* R_h . (r * h) */
          ph = ((xw[nh] + rech) + wbh) + rbh;
        }
        const double hh = oracle_activation(ak[1], aa[1], ab[1], clipv(ph, p->clip));
        hn[j] = (1.0 - gz[j]) * hh + gz[j] * h[j];
      }
    } else {
      for (int64_t j = 0; j < H; ++j) {
        double pre = ((xw[j] + rec[j]) + (Wb ? Wb[j] : 0.0)) + (Rb ? Rb[j] : 0.0);
        hn[j] = oracle_activation(ak[0], aa[0], ab[0], clipv(pre, p->clip));
      }
    }
    for (int64_t j = 0; j < H; ++j) {
      h[j] = hn[j];
      if (p->cell == OR_LSTM) c[j] = cn[j];
    }
    if (Y) {
      double* y = Y + (p->layout == 0 ? ((t * D + d) * B + b) * H : ((b * S + t) * D + d) * H);
      for (int64_t j = 0; j < H; ++j) y[j] = h[j];
    }
  }
  /* Y is zero at the steps past the length */
  if (Y)
    for (int64_t t = L; t < S; ++t) {
      double* y = Y + (p->layout == 0 ? ((t * D + d) * B + b) * H : ((b * S + t) * D + d) * H);
      for (int64_t j = 0; j < H; ++j) y[j] = 0.0;
    }
  /* a row of length 0 has zero final states; otherwise the state after its last step */
  for (int64_t j = 0; j < H; ++j) {
    if (Y_h) Y_h[sidx + j] = L == 0 ? 0.0 : h[j];
    if (Y_c) Y_c[sidx + j] = L == 0 ? 0.0 : c[j];
  }
}

/* Run a whole layer.  Any of B, lens, init_h, init_c, P may be NULL (ONNX
 * defaults: zero bias, full lengths, zero initial states, no peepholes);
 * any of Y, Y_h, Y_c may be NULL (not written).  Returns the number of
 * threads used, or a negative value on a bad argument. */
int oracle_rnn(const oracle_problem* p, const double* X, const double* W, const double* R,
               const double* Bias, const int32_t* lens, const double* init_h, const double* init_c,
               const double* P, double* Y, double* Y_h, double* Y_c, int nthreads) {
  if (!p || p->seq < 0 || p->batch < 0 || p->input < 0 || p->hidden < 0) return -1;
  if (p->cell < OR_RNN || p->cell > OR_LSTM) return -1;
  const int64_t D = p->direction == OR_BIDIRECTIONAL ? 2 : 1;
  const int64_t H = p->hidden;
  const int G = gates_of(p->cell);
  const int64_t nwork = 7 * H + 2 * (int64_t)G * H;   /* h c hn cn rh gz gr + xw rec */
  const int64_t total = D * p->batch;
  int used = 1;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  if (nthreads > total) nthreads = (int)(total > 0 ? total : 1);
  used = nthreads;
#pragma omp parallel num_threads(nthreads)
#endif
  {
    double* work = (double*)malloc(sizeof(double) * (size_t)(nwork > 0 ? nwork : 1));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t q = 0; q < total; ++q) {
      const int64_t d = q / (p->batch > 0 ? p->batch : 1);
      const int64_t b = q % (p->batch > 0 ? p->batch : 1);
      run_sequence(p, d, b, X, W, R, Bias, lens, init_h, init_c, P, Y, Y_h, Y_c, work);
    }
    free(work);
  }
  (void)nthreads;
  return used;
}
