/* Plain C oracle of the decode-time gate/up path, reading the packed blobs.
 *
 * Test infrastructure only: the tests and the benchmark's CPU baseline load
 * it (through oracle/ref_c.py); the HIP library never links or calls it, and
 * it shares no code, header or table with the library.
 *
 * Sources (BitsMoE blog note, "Methodology"):
 *   first split  - with P = U Sigma, W_e x = P (Phi^T x): z = Phi^T x is
 *                  formed once per token and shared by its experts;
 *   second split - W_e = sum_k a_{e,k} p_{e,k} phi_k^T with only p quantized,
 *                  so y_e = sum over k with b_{e,k} > 0 of a_{e,k} z_k p_hat;
 *   execution    - columns of one width stored together, bit plane by bit
 *                  plane: p_hat is read back code by code from the planes.
 * Gated MLP: h = SiLU(y_gate) * y_up with SiLU(v) = v / (1 + exp(-v)).
 * p_hat = m + s q in double (1..8-bit columns: fp16 scale s and offset m),
 * the stored fp16 value (16-bit columns).  The blob layout (format v3) is the
 * one written out in oracle/fmt.py's module text.
 *
 * Arithmetic: double throughout; z_n sums over i ascending; y sums over k
 * ascending, one term (a_k z_k) * p_hat_k[i] at a time (the order of
 * oracle/path.py).  Built with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { kHeader = 128, kDirRec = 64, kSegRows = 32, kGroups = 7, kGroupSlots = 32 };
static const int kWidth[kGroups] = {1, 2, 3, 4, 6, 8, 16};

static uint16_t rd16(const uint8_t* p) { uint16_t v; memcpy(&v, p, 2); return v; }
static uint32_t rd32(const uint8_t* p) { uint32_t v; memcpy(&v, p, 4); return v; }
static uint64_t rd64(const uint8_t* p) { uint64_t v; memcpy(&v, p, 8); return v; }
static float rdf32(const uint8_t* p) { float v; memcpy(&v, p, 4); return v; }

/* IEEE 754 binary16 -> double, from the encoding: sign, 5-bit exponent
 * (bias 15), 10-bit fraction; exponent 0 is subnormal, 31 inf/NaN. */
static double half_to_double(uint16_t h) {
  const int sign = h >> 15, ex = (h >> 10) & 31, fr = h & 1023;
  double v;
  if (ex == 0)
    v = ldexp((double)fr, -24);
  else if (ex == 31)
    v = fr ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + fr), ex - 25);
  return sign ? -v : v;
}

/* One expert of one blob, located and checked. */
typedef struct {
  const uint8_t* blk;
  const uint8_t* planes;
  uint32_t seg_words, n_seg;
  uint32_t cnt[kGroups], nb[kGroups];
  uint32_t slot0[kGroups], word0[kGroups]; /* first slot / word of each group */
  uint32_t a_off, s_off, m_off, n_slot, n_qslot;
} Expert;

static int locate(const uint8_t* blob, size_t nbytes, int E, int dout, int r, int e, Expert* x) {
  if (nbytes < kHeader || memcmp(blob, "BMOE", 4) != 0 || rd32(blob + 4) != 4) return -1;
  if ((int)rd32(blob + 8) != E || (int)rd32(blob + 12) != dout || (int)rd32(blob + 16) != r)
    return -1;
  if (e < 0 || e >= E) return -1;
  const uint64_t dir = rd64(blob + 40);
  if (dir + (uint64_t)kDirRec * E > nbytes) return -1;
  const uint8_t* d = blob + dir + (uint64_t)kDirRec * e;
  const uint64_t base = rd64(d);
  const uint64_t block_bytes = rd32(d + 44);
  if (base > nbytes || block_bytes > nbytes - base) return -1;
  x->blk = blob + base;
  x->n_seg = (uint32_t)((dout + kSegRows - 1) / kSegRows);
  x->seg_words = rd32(d + 20);
  x->a_off = rd32(d + 24);
  x->s_off = rd32(d + 28);
  x->m_off = rd32(d + 32);
  uint32_t slot = 0, word = 0, qslots = 0;
  for (int g = 0; g < kGroups; ++g) {
    x->cnt[g] = rd16(d + 48 + 2 * g);
    x->nb[g] = (x->cnt[g] + kGroupSlots - 1) / kGroupSlots * (kGroupSlots / 4);
    x->slot0[g] = slot;
    x->word0[g] = word;
    slot += 4 * x->nb[g];
    word += 4 * x->nb[g] * (uint32_t)kWidth[g];
    if (kWidth[g] < 16) qslots = slot;
  }
  x->n_slot = slot;
  x->n_qslot = qslots;
  if (word != x->seg_words) return -1;
  const uint64_t pend = (uint64_t)rd32(d + 36) + 4ull * x->n_seg * x->seg_words;
  if (pend > block_bytes) return -1;
  x->planes = x->blk + rd32(d + 36);
  return 0;
}

/* Code (1..8 bits) or fp16 bit pattern (16 bits) of output row `row` in slot
 * `s` of group g, read from the planes. */
static uint32_t code_at(const Expert* x, int g, uint32_t s, int row) {
  const int w = kWidth[g];
  const uint32_t beta = s / 4, u = s % 4;
  const int sg = row / kSegRows, oc = (row % kSegRows) / 8, rho = row % 8;
  const uint8_t* blk =
      x->planes + 4ull * ((uint64_t)sg * x->seg_words + x->word0[g] + 4ull * beta * w);
  if (w == 16) {
    const uint32_t wv = rd32(blk + 4 * (16 * oc + 2 * rho + (u >> 1)));
    return (u & 1) ? (wv >> 16) : (wv & 0xFFFFu);
  }
  uint32_t q = 0;
  for (int j = 0; j < w; ++j) {
    const uint32_t wv = rd32(blk + 4 * (w * oc + j));
    q |= ((wv >> (8 * u + rho)) & 1u) << j;
  }
  return q;
}

/* codes[k * dout + i]: the code of column k (0 for 0-bit columns), read back
 * from expert e's planes.  Returns 0, or -1 when the blob does not check. */
int bref_unpack_expert(const uint8_t* blob, size_t nbytes, int E, int dout, int r, int e,
                       uint16_t* codes) {
  Expert x;
  if (locate(blob, nbytes, E, dout, r, e, &x)) return -1;
  memset(codes, 0, sizeof(uint16_t) * (size_t)r * dout);
  for (int g = 0; g < kGroups; ++g)
    for (uint32_t s = 0; s < x.cnt[g]; ++s) {
      const uint32_t k = rd16(x.blk + 2ull * (x.slot0[g] + s));
      if (k >= (uint32_t)r) return -1;
      for (int i = 0; i < dout; ++i) codes[(size_t)k * dout + i] = (uint16_t)code_at(&x, g, s, i);
    }
  return 0;
}

/* y[i] = sum over k ascending with b_k > 0 of (a_k z_k) * p_hat_k[i]. */
static int expert_y(const Expert* x, int dout, int r, const double* z, double* y, int* slot_of_k,
                    int* group_of_k) {
  for (int k = 0; k < r; ++k) slot_of_k[k] = -1;
  for (int g = 0; g < kGroups; ++g)
    for (uint32_t s = 0; s < x->cnt[g]; ++s) {
      const uint32_t k = rd16(x->blk + 2ull * (x->slot0[g] + s));
      if (k >= (uint32_t)r || slot_of_k[k] >= 0) return -1;
      slot_of_k[k] = (int)s;
      group_of_k[k] = g;
    }
  for (int i = 0; i < dout; ++i) y[i] = 0.0;
  for (int k = 0; k < r; ++k) {
    if (slot_of_k[k] < 0) continue;
    const int g = group_of_k[k];
    const uint32_t s = (uint32_t)slot_of_k[k], gs = x->slot0[g] + s;
    const double c = (double)rdf32(x->blk + x->a_off + 4ull * gs) * z[k];
    if (kWidth[g] == 16) {
      for (int i = 0; i < dout; ++i)
        y[i] += c * half_to_double((uint16_t)code_at(x, g, s, i));
    } else {
      const double sc = half_to_double(rd16(x->blk + x->s_off + 2ull * gs));
      const double mc = half_to_double(rd16(x->blk + x->m_off + 2ull * gs));
      for (int i = 0; i < dout; ++i) y[i] += c * (mc + sc * (double)code_at(x, g, s, i));
    }
  }
  return 0;
}

/* Gate/up for T tokens.  phi_t: 2r x din fp16 (rows 0..r-1 Phi_gate^T, rows
 * r..2r-1 Phi_up^T); x: T x din fp16; ids: T x k; h: T x k x dout doubles
 * (NaN rows for an id outside [0, E) or a blob that does not check).
 * nthreads: OpenMP threads over tokens (z) and pairs (y, h); 1 = serial.
 * Returns 0, or -1 on a memory allocation failure. */
int bref_gateup(const uint8_t* blob_g, size_t bytes_g, const uint8_t* blob_u, size_t bytes_u,
                const uint16_t* phi_t, const uint16_t* x, const int32_t* ids, int T, int k,
                int E, int din, int dout, int r, int nthreads, double* h) {
  const int R = 2 * r;
  double* z = (double*)malloc(sizeof(double) * (size_t)T * R);
  if (!z) return -1;
  int fail = 0;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int t = 0; t < T; ++t)
    for (int n = 0; n < R; ++n) {
      double acc = 0.0;
      for (int i = 0; i < din; ++i)
        acc += half_to_double(phi_t[(size_t)n * din + i]) *
               half_to_double(x[(size_t)t * din + i]);
      z[(size_t)t * R + n] = acc;
    }
#pragma omp parallel num_threads(nthreads)
  {
    double* yg = (double*)malloc(sizeof(double) * (size_t)dout);
    double* yu = (double*)malloc(sizeof(double) * (size_t)dout);
    int* sk = (int*)malloc(sizeof(int) * (size_t)r);
    int* gk = (int*)malloc(sizeof(int) * (size_t)r);
    if (!yg || !yu || !sk || !gk) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int p = 0; p < T * k; ++p) {
        const int t = p / k, e = ids[p];
        double* hp = h + (size_t)p * dout;
        Expert xg, xu;
        int bad = e < 0 || e >= E || locate(blob_g, bytes_g, E, dout, r, e, &xg) ||
                  locate(blob_u, bytes_u, E, dout, r, e, &xu);
        if (!bad) bad = expert_y(&xg, dout, r, z + (size_t)t * R, yg, sk, gk) ||
                        expert_y(&xu, dout, r, z + (size_t)t * R + r, yu, sk, gk);
        for (int i = 0; i < dout; ++i)
          hp[i] = bad ? NAN : (yg[i] / (1.0 + exp(-yg[i]))) * yu[i];
      }
    }
    free(yg);
    free(yu);
    free(sk);
    free(gk);
  }
  free(z);
  return fail ? -1 : 0;
}
