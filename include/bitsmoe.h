/*
 * bitsmoe.h -- C ABI of the spectral MoE gate/up decode library (gfx950).
 *
 * The method (BitsMoE; blog note "BitsMoE: Cost-Aware Bit Allocation In
 * spectral Space for MoE LLM Quantization", section Methodology):
 *   - "first split": one SVD of the stacked expert matrices of a linear type
 *     gives a basis Phi shared by all experts, and W_e x = P_e (Phi^T x); the
 *     bracket z = Phi^T x does not depend on the expert, so the experts a
 *     token selects all reuse it.
 *   - "second split": W_e = sum_k a_{e,k} p_{e,k} phi_k^T with unit columns
 *     p_{e,k}; the magnitude a is kept, the direction p is quantized.
 *   - "Usage": per-column widths {0,1,2,3,4,6,8,16}; 0 drops the column, 16
 *     keeps it as FP16.
 *   - "execution": columns of the same width are grouped and stored by bit
 *     plane so the GPU processes the mixed widths regularly.
 * For token t routed to expert e (slot j of its top-k list) the library
 * computes
 *   y_e = sum_{k: b_{e,k} > 0} a_{e,k} z_k p_hat_{e,k},   z = Phi^T x_t,
 *   h[t, j, :] = SiLU(y_gate,e) * y_up,e,   SiLU(v) = v / (1 + exp(-v)),
 * where p_hat is the dequantized direction: m + s*q for 1..8-bit columns
 * (uniform asymmetric codes q, fp16 scale s and fp16 offset m per column),
 * the fp16 value for 16-bit columns.  Routing weights are not applied.
 *
 * Conventions for every call below:
 *   - Return value: BITSMOE_OK (0) or a negative status; bitsmoe_strerror()
 *     names it and bitsmoe_last_error_detail() gives a thread-local message.
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     allocates no device memory (bitsmoe_moe_gateup_noalloc's static array
 *     is part of the loaded code object) and never synchronizes.
 *   - Device pointers must be 16-byte aligned (ids: 4-byte aligned).
 *   - Device calls enqueue work on `stream` (0 = null stream) and return at
 *     once; inputs must stay valid until the stream reaches the work.  Host
 *     argument checks happen before anything is enqueued; a failing check
 *     enqueues nothing.
 *   - Device-side faults the host cannot see (a blob whose header does not
 *     match the dimensions passed, an expert id outside [0, E)) never cause
 *     an out-of-bounds access: the affected output rows are written as NaN.
 *   - The library keeps no state between calls except what the caller's
 *     workspace holds (bitsmoe_moe_gateup keeps a launch counter there), the
 *     static workspace of bitsmoe_moe_gateup_noalloc and the test hook's
 *     wait limit; entry points are re-entrant, and calls that share a
 *     workspace must not overlap in time.
 */
#ifndef BITSMOE_H
#define BITSMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* bitsmoe_stream_t; /* same type as hipStream_t */

#define BITSMOE_OK        0
#define BITSMOE_EINVAL   -1  /* null or misaligned pointer, T < 1, k < 1, k > E */
#define BITSMOE_ESHAPE   -2  /* non-positive dims, r > 65535, din % 8 != 0, mismatch */
#define BITSMOE_EBITS    -3  /* a width outside {0,1,2,3,4,6,8,16}, non-finite p */
#define BITSMOE_ENOSPC   -4  /* output, blob or workspace buffer too small */
#define BITSMOE_EFORMAT  -5  /* blob magic, version, CRC or directory invalid */
#define BITSMOE_EHIP     -6  /* HIP runtime or launch error */

#define BITSMOE_FORMAT_VERSION 4

/* Library version (major*10000 + minor*100 + patch). */
int bitsmoe_version(void);
const char* bitsmoe_strerror(int status);
const char* bitsmoe_last_error_detail(void);

/* ---------------------------------------------------------------- packing
 * Host-only, offline.  Quantizes and packs one linear type (gate or up) of
 * one layer ("second split", "Usage", "execution").
 *   p    : E*r*dout float32, column (e,k) at p[(e*r + k)*dout + i], unit norm
 *          expected (any finite values with |p| <= 60000 are accepted)
 *   a    : E*r float32 magnitudes a_{e,k} (stored unquantized)
 *   bits : E*r uint8 widths in {0,1,2,3,4,6,8,16}
 * Quantizer (1..8 bits), all in IEEE float32 without fused operations:
 *   s = fp16_rne((max p - min p) / (2^b - 1)), s = 1 if it rounds to 0;
 *   m = fp16_rne(min p) (-0 below +0); q_i = clamp(nearbyint((p_i - m) / s),
 *   0, 2^b - 1)
 *   with ties to even.  16 bits: fp16_rne(p_i).  0 bits: no entry.
 * Blob layout (format v4, little-endian, offsets from the blob base):
 *   header 128 B: "BMOE", u32 version(=4), E, dout, r, dout_pad
 *     (=32*ceil(dout/32)), n_seg (=dout_pad/32), header_bytes(=128);
 *     u64 total_bytes at 32, u64 dir_offset(=128) at 40, u32 CRC-32 (IEEE)
 *     of [128, total) at 48, u64 ctab_offset (=align256(128 + 64 E)) at 56.
 *   directory: E records of 64 B: u64 block_offset; u32 n_nz, n_q, n_16,
 *     seg_words (u32 words of one 32-row segment record), a_off, s_off,
 *     m_off, planes_off; f32 cmax (largest |a|*s over 1..8-bit columns,
 *     |a| over 16-bit ones); u32 block_bytes; u16 count[7] of widths
 *     1,2,3,4,6,8,16 at 48 (offsets relative to the expert block).
 *   component table at ctab_offset: per expert, at stride
 *     ctab_stride = 3 align16(2 r) + align16(4 r) + 16, the expert's
 *     components in k order (it lets whoever holds z_k form the coefficient
 *     of every routed expert without the directory): u16 slot[r] (slot of
 *     component k in the expert's slot order, 0xFFFF for a 0-bit
 *     component: the inverse of kidx) @0, f16 s[r] @align16(2 r), f16 m[r]
 *     @2 align16(2 r) (both 0 for 16- and 0-bit components), f32 a[r]
 *     @3 align16(2 r) (0 for 0-bit ones), f32 cmax (the directory's) and 12
 *     zero bytes @3 align16(2 r) + align16(4 r).  bitsmoe_blob_check
 *     rebuilds every expert's table from its block and compares bytes.
 *   expert block (256-aligned, back to back from
 *     align256(ctab_offset + E ctab_stride)): slots ordered by width group
 *     1,2,3,4,6,8,16, ascending k inside a group, each group padded with
 *     zero slots to a multiple of 32 (so a 32-slot step has one width);
 *     0-bit columns have no slot.  n_slot slots, n_qslot of width <= 8:
 *     u16 kidx[n_slot] @0, f32 a[n_slot] @a_off, f16 s[n_qslot] @s_off,
 *     f16 m[n_qslot] @m_off (padding slots: all 0), then
 *     u32 planes[n_seg][seg_words] @planes_off: one record per 32 output
 *     rows; in it, 4-slot block after block, 4*w words per block of width
 *     w: for row octet i = 0..3, w words.  w <= 8: word (i, j) is plane j,
 *     its bit 8*u + rho is bit j of the code of row 8i + rho in slot u of
 *     the block (byte u holds the octet's 8 rows of slot u).  w = 16: word
 *     (i, 2*rho + h) holds the fp16 values of row 8i + rho in slots 2h
 *     (low half) and 2h + 1.  Rows >= dout are 0.
 *   block_bytes = align256(planes_off + 4*n_seg*seg_words + 16); all
 *     padding bytes are zero.
 * bitsmoe_pack_size: bytes the blob needs.  bitsmoe_pack: writes it into the
 * host buffer `out` (out_bytes >= that size, else BITSMOE_ENOSPC).
 */
int bitsmoe_pack_size(int E, int dout, int r, const uint8_t* bits, size_t* out_bytes);
int bitsmoe_pack(int E, int dout, int r, const float* p, const float* a,
                 const uint8_t* bits, void* out, size_t out_bytes);

/* Device packer: the same blob bytes as bitsmoe_pack, produced on the GPU
 * ("second split", "Usage", "execution").
 *   p, a : device float32 arrays laid out as for bitsmoe_pack
 *   bits : HOST array of E*r widths (the layout is planned on the host)
 *   out  : device buffer of out_bytes >= bitsmoe_pack_size() bytes, 16-byte
 *          aligned; on success it holds the complete blob (header and CRC
 *          included)
 *   ws   : device workspace of >= bitsmoe_pack_device_workspace_size()
 *          bytes, 16-byte aligned (slot table, checksum chunks, flags)
 * The quantizer is the one above, in IEEE float32 without contraction, so
 * the codes match the host packer's bit for bit; the CRC is taken over 4 KiB
 * chunks on the device and folded on the host.  Work is issued on `stream`
 * and the call returns after synchronizing it (the host folds the checksum
 * and reads the validation flags).  BITSMOE_EBITS for a non-finite a or a
 * stored p that is not finite or has |p| > 60000 (out is then unspecified);
 * E must not exceed 65535. */
int bitsmoe_pack_device_workspace_size(int E, int dout, int r, const uint8_t* bits,
                                       size_t* bytes);
int bitsmoe_pack_device(int E, int dout, int r, const float* p, const float* a,
                        const uint8_t* bits, void* out, size_t out_bytes, void* ws,
                        size_t ws_bytes, bitsmoe_stream_t stream);

/* ------------------------------------------------------------------ FQCM
 * Inputs of the width allocation (BitsMoE blog note, Methodology: the FQCM
 * importance, loss and marginal gain; "Usage": widths chosen jointly under a
 * bit budget).  All arrays are device memory.
 *
 * bitsmoe_fqcm_distortion: eps[(e*r + k)*8 + i] (float64) for the widths
 *   (0,1,2,3,4,6,8,16)[i] of column p_{e,k} (p laid out as for bitsmoe_pack):
 *   eps(0) = ||p||^2, eps(b) = ||p - (m + s q)||^2 with the quantizer above,
 *   eps(16) = ||p - fp16(p)||^2; float64 sums.  Async on `stream`.
 * bitsmoe_fqcm_beta: beta[e*r + k] = sum over the pairs (t, j) with
 *   ids[t*k + j] = e, in that order, of g[t*k + j] * z[t*z_stride + k]^2
 *   (float64; z = Phi^T x of T calibration tokens, e.g. from
 *   bitsmoe_spectral_proj; g: float32 routing weights; pairs whose id is
 *   outside [0, E) are skipped).  Async on `stream`.
 * bitsmoe_fqcm_allocate: widths bits[e*r + k] (device uint8) minimising
 *   sum L(b) with L(b) = ((a*a)*beta)*eps(b) (float64) subject to
 *   sum dout*b <= budget_bits: the integer program's exact minimum (ties to
 *   the narrower width, then to the fewest bits; float64 sums, so two
 *   allocations whose losses differ only by rounding may be taken either
 *   way).  Steps: the Lagrangian relaxation (each column minimises
 *   L(b) + lam*(dout*b), ties to the narrower width, at the smallest double
 *   lam >= 0 whose total fits: bisection over the bit patterns of doubles),
 *   then an exact step over the columns whose reduced cost at lam is within
 *   the gap to the dual bound.  *used_bits <= budget_bits gets the bits
 *   used, *lambda lam, *lp_gap the loss minus the dual bound
 *   D(lam) = sum_c min_b (L_c(b) + lam*dout*b) - lam*dout*floor(budget/dout)
 *   (0 when the Lagrangian widths use the whole budget; any pointer may be
 *   NULL).  BITSMOE_ENOSPC when more than 65536 alternatives, or more than
 *   2^28 column x unit states, fall within that gap (not seen on the
 *   synthetic layers).  ws: device memory of BITSMOE_FQCM_WS_BYTES bytes,
 *   8-byte aligned.  The call synchronizes `stream` once per bisection step
 *   (at most 65 + 64 steps) and runs the exact step on the host.
 */
#define BITSMOE_FQCM_WS_BYTES ((size_t)1024 + 65536 * 24)
int bitsmoe_fqcm_distortion(const float* p, int E, int r, int dout, double* eps,
                            bitsmoe_stream_t stream);
int bitsmoe_fqcm_beta(const float* z, int z_stride, const int32_t* ids, const float* g, int T,
                      int k, int E, int r, double* beta, bitsmoe_stream_t stream);
int bitsmoe_fqcm_allocate(const float* a, const double* beta, const double* eps, int E, int r,
                          int dout, uint64_t budget_bits, uint8_t* bits, double* lambda,
                          uint64_t* used_bits, double* lp_gap, void* ws, size_t ws_bytes,
                          bitsmoe_stream_t stream);

/* Host-side check of a blob in host memory: magic, version, sizes, CRC and
 * every directory record.  Fills E, dout, r when the pointers are non-null.
 * BITSMOE_EFORMAT on any inconsistency. */
int bitsmoe_blob_check(const void* blob, size_t bytes, int* E, int* dout, int* r);

/* --------------------------------------------------------- shared projection
 * z = Phi^T x for every token ("first split": computed once per token and
 * shared by all routed experts).
 *   phi_t_f16 : r_total*din fp16, basis vector n at phi_t_f16[n*din .. +din)
 *               (Phi stored transposed: row n is phi_n).  Gate and up bases
 *               may be stacked as r_total = 2r rows.
 *   x_f16     : T*din fp16 activations, token t at x[t*din]
 *   z         : T*r_total float32 output, z[t*r_total + n]
 * din must be a multiple of 8.  fp16 products are exact in float32 and are
 * accumulated in float32. */
int bitsmoe_spectral_proj(const void* phi_t_f16, const void* x_f16, float* z,
                          int T, int din, int r_total, bitsmoe_stream_t stream);

/* ------------------------------------------------------------ expert apply
 * One linear type, no epilogue: for every pair (t, j), e = ids[t*k + j],
 *   y[(t*k + j)*dout + i] = sum_{k: b>0} a_{e,k} z[t*z_stride + k] p_hat_{e,k}[i]
 * ("second split").  packed: device copy of a bitsmoe_pack blob of
 * packed_bytes bytes for (E, dout, r).  z: T rows of z_stride >= r floats.
 * ws/ws_bytes: may be NULL/0 (no workspace needed). */
int bitsmoe_expert_apply(const void* packed, size_t packed_bytes, int E, int dout,
                         int r, const float* z, int z_stride, const int32_t* ids,
                         int T, int k, float* y, void* ws, size_t ws_bytes,
                         bitsmoe_stream_t stream);

/* ------------------------------------------------------------ full gate/up
 * h[(t*k + j)*dout + i] = SiLU(y_gate)[i] * y_up[i] for e = ids[t*k + j].
 *   packed_gate / packed_up : device blobs of gate_bytes / up_bytes
 *   phi_t_gateup_f16        : 2r*din fp16: rows 0..r-1 = Phi_gate^T,
 *                             rows r..2r-1 = Phi_up^T
 *   x_f16 : T*din fp16; ids : T*k int32; h : T*k*dout float32
 *   ws    : device workspace of at least bitsmoe_moe_gateup_workspace_size()
 *           bytes, zero-filled once before its first use
 *           (bitsmoe_workspace_init).  The one-launch path (T <= 4) keeps a
 *           launch counter and cumulative hint counters in its first 8448
 *           bytes from call to call (at that fixed place whatever T is, so
 *           one workspace, sized for the largest T, may serve calls of any T
 *           in turn); calls that share a workspace must not run concurrently.
 * At T = 1 (k <= 16, r <= 2048 and a multiple of 4, din <= 2048) one launch
 * also forms every routed expert's coefficients next to z.  Their integer
 * scale comes from the blob's bound cmax and |z_k| <= ||x||_2, which holds
 * for the unit-norm rows of a basis from a factorization; rows of Phi^T
 * whose norm exceeds 1.86 can push a coefficient past the scale, and the
 * affected rows of h are then NaN (never out-of-bounds accesses).
 */
int bitsmoe_moe_gateup_workspace_size(int T, int k, int E, int din, int dout, int r,
                                      size_t* bytes);
int bitsmoe_moe_gateup(const void* packed_gate, size_t gate_bytes,
                       const void* packed_up, size_t up_bytes,
                       const void* phi_t_gateup_f16, const void* x_f16,
                       const int32_t* ids, int T, int k, int E, int din, int dout,
                       int r, float* h, void* ws, size_t ws_bytes,
                       bitsmoe_stream_t stream);

/* ------------------------------------------------- gate/up, no allocation
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): bitsmoe_moe_gateup
 * with the same arguments, meanings and results, minus the workspace.  The
 * workspace is a static array of BITSMOE_GATEUP_NOALLOC_MAX_WS bytes in the
 * library's device code, one per device, which the device keeps until the
 * process ends; the first call on a device zero-fills it on `stream`.
 *   - A call whose bitsmoe_moe_gateup_workspace_size() exceeds that size
 *     returns BITSMOE_ENOSPC and enqueues nothing.
 *   - Calls no hipMalloc, hipFree or other allocating routine.
 *   - Every call on one device shares that array: calls that overlap in
 *     time on one device (other streams, other threads) race and must not
 *     be made; calls in order on one stream are fine.
 */
#define BITSMOE_GATEUP_NOALLOC_MAX_WS ((size_t)64 << 20)
int bitsmoe_moe_gateup_noalloc(const void* packed_gate, size_t gate_bytes,
                               const void* packed_up, size_t up_bytes,
                               const void* phi_t_gateup_f16, const void* x_f16,
                               const int32_t* ids, int T, int k, int E, int din,
                               int dout, int r, float* h, bitsmoe_stream_t stream);

/* ---------------------------------------------------------- down + combine
 * out[t*din + i] = sum over slots j (ascending) of g[t*k + j] * y_{t,j}[i],
 *   y_{t,j} = sum_{c: b>0} a_{e,c} z_c p_hat_{e,c},  z = Phi_down^T fp16(h_{t,j}),
 *   e = ids[t*k + j]; a pair whose id is outside [0, E) contributes nothing.
 * The down projection with the same two splits as gate/up (BitsMoE blog
 * note, Methodology); its basis lives in the input space of down_proj, so z
 * is formed per (token, slot) from that pair's h.
 *   packed_down      : device blob (bitsmoe_pack with rows = din, r = r_d)
 *   phi_t_down_f16   : r_d*dout fp16, row c = phi_c (Phi_down transposed)
 *   h                : T*k*dout float32 (the gate/up output), rounded to fp16
 *   ids, g           : T*k int32 expert ids and float32 routing weights
 *   out              : T*din float32
 *   ws               : >= bitsmoe_moe_down_workspace_size() bytes, 256-byte
 *                      aligned (fp16 h, z and the per-pair outputs)
 * dout must be a multiple of 8.  Async on `stream`. */
int bitsmoe_moe_down_workspace_size(int T, int k, int E, int dout, int din, int r_d,
                                    size_t* bytes);
int bitsmoe_moe_down(const void* packed_down, size_t down_bytes, const void* phi_t_down_f16,
                     const float* h, const int32_t* ids, const float* g, int T, int k, int E,
                     int dout, int din, int r_d, float* out, void* ws, size_t ws_bytes,
                     bitsmoe_stream_t stream);

/* ------------------------------------------------------------------- SSD
 * Shared-basis spectral decomposition of one linear type (BitsMoE blog note,
 * Methodology, first and second split): W_cat = [W_1; ...; W_E] =
 * U Sigma Phi^T, P = U Sigma, W_e = sum_k a_{e,k} p_{e,k} phi_k^T.
 *   W     : device E*dout*din float32, W_e row-major at W[e*dout*din]
 *   phi   : device din*r float32 (phi_k = column k), the r leading right
 *           singular vectors, each signed so that its first largest-magnitude
 *           entry is positive
 *   a, p  : device E*r and E*r*dout float32 (p laid out as for bitsmoe_pack;
 *           a zero column gets p = e_0)
 *   sigma2: optional HOST array of r float64 squared singular values
 *   sweeps: optional HOST int, the Jacobi sweeps taken
 * Float64 Gram matrix and cyclic Jacobi (circle ordering) until the
 * off-diagonal mass is below (1e-15 ||G||)^2 or max_sweeps sweeps.  ws: device
 * memory of bitsmoe_ssd_workspace_size() bytes, 256-byte aligned.  The call
 * synchronizes `stream` (once per sweep and at the end).  din <= 8192,
 * r <= min(din, E*dout). */
int bitsmoe_ssd_workspace_size(int E, int dout, int din, int r, size_t* bytes);
int bitsmoe_ssd(const float* W, int E, int dout, int din, int r, float* phi, float* a, float* p,
                double* sigma2, int* sweeps, int max_sweeps, void* ws, size_t ws_bytes,
                bitsmoe_stream_t stream);

/* Zero-fills a workspace with a kernel (no memset node), on `stream`. */
int bitsmoe_workspace_init(void* ws, size_t ws_bytes, bitsmoe_stream_t stream);

/* ---------------------------------------------------------------- testing
 * bitsmoe_debug_set_wait_limit: sets the bound on the one-launch gate/up
 * kernel's waits for z produced by its other work-groups (default 2^20
 * re-reads; 0 gives up at once, so every row of the launch becomes NaN and
 * every work-group still exits) and returns the previous bound.  Process-wide;
 * for tests of the give-up path. */
uint32_t bitsmoe_debug_set_wait_limit(uint32_t spins);

/*
 * bitsmoe_wait_timeouts: the number of waits of the one-launch gate/up
 * kernels (bitsmoe_moe_gateup at T <= 4) that gave up since the workspace
 * was zero-filled, cumulative over calls.  Those kernels need every
 * work-group resident at once (the groups wait for each other's z); when
 * another kernel or process holds compute units, a wait can run out its
 * bound, and the rows it covers are written as NaN while the call itself
 * still returns BITSMOE_OK.  A count that grew across a call says that this
 * happened.  ws / ws_bytes: the workspace the calls used (device memory);
 * ws = NULL reads the current device's static workspace of
 * bitsmoe_moe_gateup_noalloc.  count: host pointer, receives the count.
 * Synchronises `stream` (the count includes every call queued on it).
 * Returns BITSMOE_EINVAL for a null count or a workspace smaller than its
 * sync words, BITSMOE_EHIP when the copy fails.
 */
int bitsmoe_wait_timeouts(const void* ws, size_t ws_bytes, uint32_t* count,
                          bitsmoe_stream_t stream);

/*
 * Codes of expert e as one of the device decoders produces them, in k order
 * ("execution": the width-grouped plane layout read back), for bit-exact
 * tests of the decode each kernel actually runs.  codes: device buffer of
 * r*dout uint16, 16-byte aligned; 0-bit columns are 0; a directory record
 * that fails its check gives 0xFFFF everywhere.  codes[k*dout + i] is
 *   path BITSMOE_DUMP_I8  : the int8 A-operand byte of the one-launch
 *                           kernel's apply (q for 1..6-bit columns, q ^ 0x80
 *                           for 8-bit ones), the fp16 bit pattern of 16-bit
 *                           columns;
 *   path BITSMOE_DUMP_F16 : the fp16 A operand of the batched kernel's apply
 *                           (the fp16 bit pattern of q, or of the stored
 *                           value for 16-bit columns);
 *   path BITSMOE_DUMP_LANE: q (1..8-bit), the fp16 bit pattern (16-bit), as
 *                           read by the lane-per-row kernel of
 *                           bitsmoe_expert_apply and of gate/up beyond the
 *                           MFMA kernels' limits.
 * A path outside these returns BITSMOE_EINVAL. */
#define BITSMOE_DUMP_I8   0
#define BITSMOE_DUMP_F16  1
#define BITSMOE_DUMP_LANE 2
int bitsmoe_dump_codes(const void* packed, size_t packed_bytes, int E, int dout,
                       int r, int e, int path, uint16_t* codes,
                       bitsmoe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BITSMOE_H */
