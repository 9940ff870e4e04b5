// HIP kernels and C ABI of the speculative-decoding verification sampler,
// written for AMD CDNA4 (gfx950, MI355X).
//
// What is computed (velog "6-1편. Speculative Decoding", section 2
// "알고리즘 4단계" steps 2-4 with section 2-1, the min(1, p/q) rule, and
// section 2-2, the residual norm(max(0, p - q)); greedy rule of "How to
// Scale Your Model -- All About Transformer Inference", Appendix D): see
// include/specverify.h.
//
// A run is one launch of verify_kernel on the caller's stream (two for a
// ragged batch: layout_kernel first checks cu_draft and writes one record
// per target row plus the split of the batch into row groups).
//
// Work is split into eight row groups, one per XCD of an MI355X
// (workgroup b runs on XCD b % 8).  A group owns a contiguous range of
// whole sequences, so every row of a sequence, and every value its waves
// exchange, stays in one XCD's L2.  The grid is persistent: what the GPU
// holds at once.
//
// Streaming.  The unit of work is an item: 4 KB of one target row (a chunk
// of 2048 bf16 or 1024 fp32 logits) plus the same chunk of the draft row
// when the position has one, so p_k and q_k of a token meet in the same
// lane.  One wave owns one item at a time; wave j of a group takes items
// j, j + Gw, j + 2 Gw, ... of the group's row-major item list, so the chunks
// of a row are handled in one round by different waves.
//   phase 1   chunk max m_c (DPP), e_k = 2^(l_k s - m_c s) with s = log2(e)/T
//             kept in registers, chunk sum s_c; (m_c, s_c) of target and
//             draft go out in epoch-tagged slots.  T = 0: chunk argmax.
//   phase 2   once every chunk of the row has published: the row normalisers
//             (M, S) = merge of (m_c, s_c); with a_c = 2^((m_c - M) s) / S and
//             rho = a_d / a_t, p_k = a_t e_t and q_k = a_t rho e_d, so
//             min(p, q) = a_t min(e_t, rho e_d) and max(0, p - q) =
//             a_t (e_t - min(e_t, rho e_d)); the chunk sums of both (beta,
//             velog section 2-3 item 1; residual mass Z, item 2) go out in
//             epoch-tagged partials.
// The waves are software pipelined: a step runs phase 1 of item k + 1, then
// runs phase 2 of item k (whose row it polled as phase 1 began), with the
// 16-byte loads of item k + 2 in flight (issued into the registers that the
// unpack of item k + 1 has just freed).  Logits are read with buffer loads over one
// chunk: a row without a draft gets a zero-sized buffer, so every item
// issues the same loads and none of them touches memory it should not.
// Without draft logits (token-only drafts, q = delta_x; or no drafts at
// all) only phase 1 runs, and the chunk that holds a drafted token x also
// publishes e_t at x.
//
// Resolution.  When a workgroup has streamed its items, it resolves the
// sequences dealt to it, one at a time: its waves take the sequence's rows
// and merge that row's slots and partials (Z and beta); find the chunk
// whose CDF interval holds u_gamma * Z (or the CDF of p for the bonus row
// and when Z = 0) and re-read it; form p(x) and q(x) from the two logits of
// the drafted token (a token-only draft: e_t at x from the slots, q(x) = 1);
// test u_i q(x) < p(x); and, for a rejected row, scan the re-read chunk in
// token order for the token.  The row results meet in LDS, where one wave
// finds the sequence's first rejection n and writes accepted_len and the
// n + 1 tokens.  The accepted length never leaves the device.
//
// Draft trees (specverify_run_tree, their own instantiation of the kernel)
// stream like token-only rows; a tree's resolution loads the tree into LDS,
// forms every candidate's p under its parent's row on four waves and walks
// the tree on one wave (see resolve_tree).
//
// commit_kernel (its own call, specverify_commit) appends each sequence's
// n + 1 emitted tokens to its token row on the device.
//
// Values cross waves only in 64-bit slots and 16-byte partials that carry a
// 32-bit epoch tag next to the value.  They are written with plain stores
// (the CU's L1 writes through to the XCD's L2) and polled with loads that
// skip L1 and read that L2; the waves that meet over a row all run on one
// XCD, so a reader that sees the tag sees the value, without fences or
// atomics.  Nothing guarantees that every workgroup of the grid is resident
// at once, so a wave that has polled spin_limit times reads the chunks that
// are still missing and computes their slots and partials itself
// (bit-identical to what their owners publish); every wait therefore ends.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <new>

#include "specverify.h"

namespace {

constexpr int kStreamWaves = 4;                // waves per workgroup
constexpr int kStreamThreads = 64 * kStreamWaves;
constexpr int kU = 4;                          // 16-byte loads per lane and row of an item
constexpr int kRowBytes = kU * 64 * 16;        // bytes of one row in one item (4 KB)
constexpr int kMaxChunks = 256;                // chunks per fp32 row (V <= 262144)
constexpr int kMaxChunksBf16 = 128;            // chunks per bf16 row (V <= 262144)
constexpr int kGroups = 8;                     // row groups = XCDs of an MI355X
constexpr int kX1 = 4;                         // exchange slots per (row, chunk)
constexpr int kPart = 4;                       // floats of partials per (row, chunk)
constexpr int kMaxGamma = 255;                 // rows per sequence <= 256
constexpr size_t kScratchBytes = (size_t)16 << 20;   // the static scratch of allocation-free runs, per device
constexpr int kLayoutThreads = 1024;
constexpr int kDefaultSpin = 64;               // polls (~1 us each) before a wave computes missing chunks itself
constexpr int kMaxSpin = 1 << 20;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFltMin = 1.17549435e-38f;
constexpr float kFltMax = 3.40282347e38f;
constexpr uint32_t kTokMask = (1u << 23) - 1;
constexpr uint32_t kAccBit = 1u << 23;
constexpr uint32_t kStatusShift = 24;          // 0 ok, 1 invalid data, 2 wait expired
constexpr int kRsrcWord3 = 0x00020000;         // raw (untyped) buffer, gfx9 family
constexpr int kNT = 2;                         // buffer-load cache policy: nontemporal
constexpr int kSC1 = 16;                       // buffer-load cache policy sc1: the load misses L1 and reads L2

// Partials of one (row, chunk), kPart floats: the epoch that completed the
// item (bits), the sum of e_t - min(e_t, rho e_d), the sum of
// min(e_t, rho e_d), unused.

template <int DT> struct Fmt;
template <> struct Fmt<SPECVERIFY_F32> {
  static constexpr int EPV = 4;   // logits per 16-byte vector
  static constexpr int ESIZE = 4;
  static constexpr int L = kU * EPV;   // logits per lane and row of an item
  static constexpr int CH = 64 * L;    // logits per chunk
};
template <> struct Fmt<SPECVERIFY_BF16> {
  static constexpr int EPV = 8;
  static constexpr int ESIZE = 2;
  static constexpr int L = kU * EPV;
  static constexpr int CH = 64 * L;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

struct Params {
  const char* target;
  const char* draft;         // NULL: no draft logits in this launch
  uint32_t tstride_b;        // row strides in bytes (< 2^31)
  uint32_t dstride_b;
  const int32_t* tokens;
  const float* uniforms;
  const float* temps;
  const int32_t* cu_draft;   // NULL: uniform gamma
  const int4* rowinfo;       // ragged: per target row {sequence, draft row, has draft, T bits}
  const uint32_t* layout;    // ragged: epoch * 2 + (layout invalid)
  const int32_t* gbounds;    // ragged: [2 (kGroups + 1)] row bounds, then sequence bounds, of the groups
  int32_t grow[kGroups + 1]; // uniform gamma: first target row of each group (and R_t)
  int32_t gseq[kGroups + 1]; // uniform gamma: first sequence of each group (and B)
  int32_t gamma;
  int32_t B;
  int32_t R_d;
  int32_t R_t;
  int32_t V;
  int32_t C;                 // chunks per row
  int32_t Gw;                // waves per row group
  int32_t Wg;                // workgroups per row group
  int32_t max_gamma;
  uint32_t epoch;
  int32_t spin_limit;
  int32_t token_only;        // drafts come without logits: q_i = delta_{x_i}
  uint32_t div_c[3];         // unsigned division by C: multiplier and two shifts
  uint32_t div_g[3];         // unsigned division by gamma + 1 (uniform gamma)
  uint64_t* xch1;            // [rows][C][kX1] tagged slots
  uint64_t* dummy;           // [waves][8]: where a wave's step with nothing to publish writes
  float* part;               // [rows][C][kPart]
  int32_t* acc_len;
  int32_t* out_tokens;
  float* p_draft;
  float* q_draft;
  float* beta;
  float* resid;
  // draft trees (token-only candidates): node parents, and the extra outputs
  int32_t tree;
  const int32_t* parents;    // [R_d] parent of each drafted node, local (0 = root)
  int32_t* out_nodes;        // [R_t] accepted nodes in path order, or NULL
  float* p_cand;             // [R_d] each candidate under its parent's target distribution, or NULL
};

// ------------------------------------------------------------------ slots

// One 64-bit store (single-copy atomic); the CU's L1 writes it through to
// the XCD's L2, where the sc1 loads of the other waves of the row find it.
__device__ __forceinline__ void slot_put(uint64_t* p, uint32_t tag, uint32_t v) {
  *p = ((uint64_t)tag << 32) | v;
}
__device__ __forceinline__ uint32_t slot_tag(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float slot_f(uint64_t w) { return __uint_as_float((uint32_t)w); }

// ------------------------------------------------------------------ wave primitives (DPP)
// Reductions use a fixed order, so every wave that reduces the same data (an
// item's phase 2, a resolving wave, the help path) gets the same bits.

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float v, float fill) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL, ROW_MASK,
                                                    0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Sum over the 64 lanes: a butterfly inside each 16-lane row, then
// row_bcast:15 and row_bcast:31 fold the rows as (r3 + r2) + (r1 + r0).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror
  v += dpp<0x140>(v);   // row_mirror
  v += dpp_rows<0x142, 0xa>(v, 0.0f);   // rows 1, 3 += last lane of rows 0, 2
  v += dpp_rows<0x143, 0xc>(v, 0.0f);   // rows 2, 3 += lane 31
  return lane_f(v, 63);
}
// Max over the 64 lanes on order-preserving integer keys of the floats
// (integer max needs no NaN quieting, so each step is one DPP max); a
// positive NaN would win, which only makes an invalid row invalid.
__device__ __forceinline__ int f2key(float f) {
  const int b = __float_as_int(f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key2f(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }
template <int CTRL>
__device__ __forceinline__ int dpp_all(int v) {    // every lane has a source lane
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true);
}
// The rows' results folded as wave_sum folds them: rows 1, 3 take lane 15,
// 47, then rows 2, 3 lane 31, so lane 63 holds the result; rows a step does
// not write get `fill`, the operation's identity.
constexpr int kKeyMin = -0x7FFFFFFF - 1;
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_rows_i(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ float wave_max(float f) {
  int v = f2key(f);
  v = max(v, dpp_all<0xB1>(v));
  v = max(v, dpp_all<0x4E>(v));
  v = max(v, dpp_all<0x141>(v));
  v = max(v, dpp_all<0x140>(v));
  v = max(v, dpp_rows_i<0x142, 0xa>(v, kKeyMin));
  v = max(v, dpp_rows_i<0x143, 0xc>(v, kKeyMin));
  return key2f(__builtin_amdgcn_readlane(v, 63));
}
// Inclusive prefix sum over the 64 lanes, fixed association.
__device__ __forceinline__ float wave_scan(float v, int lane) {
  v += dpp<0x111>(v);   // row_shr:1 (bound_ctrl: 0 enters at the row start)
  v += dpp<0x112>(v);   // row_shr:2
  v += dpp<0x114>(v);   // row_shr:4
  v += dpp<0x118>(v);   // row_shr:8
  const float t0 = lane_f(v, 15), t1 = lane_f(v, 31), t2 = lane_f(v, 47);
  const float t01 = t0 + t1, t012 = t01 + t2;
  // the offset of the lane's row of 16, by selects (a chained conditional
  // here compiled to branches on the lane)
  const int row = lane >> 4;
  float off = row >= 1 ? t0 : 0.0f;
  off = row >= 2 ? t01 : off;
  off = row >= 3 ? t012 : off;
  return v + off;
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dppi<0xB1>(v));
  v = min(v, dppi<0x4E>(v));
  v = min(v, dppi<0x141>(v));
  v = min(v, dppi<0x140>(v));
  v = min(v, dpp_rows_i<0x142, 0xa>(v, 0x7FFFFFFF));
  v = min(v, dpp_rows_i<0x143, 0xc>(v, 0x7FFFFFFF));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dppi<0xB1>(v));
  v = max(v, dppi<0x4E>(v));
  v = max(v, dppi<0x141>(v));
  v = max(v, dppi<0x140>(v));
  v = max(v, dpp_rows_i<0x142, 0xa>(v, kKeyMin));
  v = max(v, dpp_rows_i<0x143, 0xc>(v, kKeyMin));
  return __builtin_amdgcn_readlane(v, 63);
}
// (value, index): larger value wins, lower index on ties.
// (v2, k2) wins over (v, k) if larger, or equal with a lower index.  Written
// without short-circuit evaluation: selects, not branches.
__device__ __forceinline__ void argmax_merge(float& v, int& k, float v2, int k2) {
  const bool take = (v2 > v) | ((v2 == v) & (k2 < k));
  v = take ? v2 : v;
  k = take ? k2 : k;
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& k) {
  const float v2 = __int_as_float(dppi<CTRL>(__float_as_int(v)));
  const int k2 = dppi<CTRL>(k);
  argmax_merge(v, k, v2, k2);
}
__device__ __forceinline__ void wave_argmax(float& v, int& k) {
  argmax_step<0xB1>(v, k);
  argmax_step<0x4E>(v, k);
  argmax_step<0x141>(v, k);
  argmax_step<0x140>(v, k);   // every lane holds its row's (max, first index)
  float bv = lane_f(v, 0);
  int bk = __builtin_amdgcn_readlane(k, 0);
#pragma unroll
  for (int l = 16; l < 64; l += 16) argmax_merge(bv, bk, lane_f(v, l), __builtin_amdgcn_readlane(k, l));
  v = bv;
  k = bk;
}

// Exponent offset of a chunk: -m s rounded, or 0 for a chunk of only -inf
// (so that its exponentials are 2^-inf = 0 instead of NaN).  A chunk's
// exponentials are e_k = 2^(l_k s + offset).
__device__ __forceinline__ float chunk_offset(float m, float s) {
  return (m == -__builtin_huge_valf()) ? 0.0f : -m * s;
}
// The offset's rounding error: -m s = chunk_offset(m, s) + chunk_lo(m, s)
// exactly (the error of a rounded product is a float, and one fma gives it
// exactly).  The e_k of the chunk carry the factor 2^-lo; the chunk's scale
// puts it back, so the offset's rounding (up to 2^-25 |m s|, a few 1e-5 at
// low temperatures) never reaches p, q, beta or Z.
__device__ __forceinline__ float chunk_lo(float m, float s) {
  return (m == -__builtin_huge_valf()) ? 0.0f : __builtin_fmaf(-m, s, -chunk_offset(m, s));
}
// Exponent of a chunk's scale against the row maximum M: (m - M) s + lo,
// so that p_k = 2^(chunk_exp) e_k / S.
__device__ __forceinline__ float chunk_exp(float m, float M, float s) {
  return __builtin_fmaf(m - M, s, chunk_lo(m, s));
}
// Scale of a chunk: p_k = scale * e_k.
__device__ __forceinline__ float chunk_scale(float m, float M, float S, float s) {
  return __builtin_amdgcn_exp2f(chunk_exp(m, M, s)) / S;
}
// rho = a_d / a_t of a chunk (q_k = a_t rho e_d), from the chunk maxima and
// the row normalisers: 2^(((m_d - M_d) - (m_t - M_t)) s + lo_d - lo_t) S_t / S_d.
// Every wave takes it from this function, so a chunk's residual weights
// e_t - min(e_t, rho e_d) have the same bits wherever they are computed.
__device__ __forceinline__ float chunk_rho(float mt, float Mt, float St, float md, float Md, float Sd, float s) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf((md - Md) - (mt - Mt), s, chunk_lo(md, s) - chunk_lo(mt, s))) *
         (St * __builtin_amdgcn_rcpf(Sd));
}
// min(a, b) of two floats that are >= 0 (+0, positive, +inf or a positive
// NaN): the unsigned order of their bit patterns is their order, NaN above
// everything, as fminf treats it.  One integer instruction; fminf would add
// a canonicalisation of each operand.
__device__ __forceinline__ float min_nonneg(float a, float b) {
  return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
}
// Weight of one logit pair in the residual, in the chunk's units: e_t minus
// min(e_t, rho e_d).
__device__ __forceinline__ float resid_w(float et, float ed, float rho) {
  return et - min_nonneg(et, rho * ed);
}


// ------------------------------------------------------------------ chunk slots and partials of a row

// The exchange slots of every chunk of row r, lane-major: lane l holds
// chunks l, l + 64, ...  Lanes past the last chunk re-read the last one,
// whose values they never use.
template <int NPER>
struct RowSlots {
  uint64_t w[NPER][kX1];
};
// Byte offsets of a lane's chunk records inside a row, `bytes` per chunk
// (loop invariant).
template <int NPER>
__device__ __forceinline__ void chunk_offsets(int C, int lane, int bytes, uint32_t (&off)[NPER]) {
#pragma unroll
  for (int j = 0; j < NPER; ++j) off[j] = (uint32_t)min(lane + 64 * j, C - 1) * (uint32_t)bytes;
}
// The slots of row r, read two at a time with 16-byte buffer loads that miss
// the CU's L1 (sc1) and are served by the XCD's L2, through a buffer over
// the row's slots: a uniform base and loop-invariant lane offsets, so no
// vector register is written before the loads issue.  `real` false: a
// zero-sized buffer, the loads read zeros (tag 0 is never an epoch) and
// touch no memory.
template <int NPER>
__device__ __forceinline__ void slots_issue(const Params& P, int r, bool real, const uint32_t (&off)[NPER],
                                            RowSlots<NPER>& q) {
  const Rsrc rs = __builtin_amdgcn_make_buffer_rsrc((void*)(P.xch1 + (int64_t)(real ? r : 0) * P.C * kX1),
                                                    (short)0, real ? P.C * kX1 * (int)sizeof(uint64_t) : 0,
                                                    kRsrcWord3);
#pragma unroll
  for (int j = 0; j < NPER; ++j)
#pragma unroll
    for (int k = 0; k < kX1; k += 2) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off[j] + k * 8, 0, kSC1);
      q.w[j][k] = (uint64_t)v[0] | ((uint64_t)v[1] << 32);
      q.w[j][k + 1] = (uint64_t)v[2] | ((uint64_t)v[3] << 32);
    }
}
// Every chunk's slots carry `tag` (wave-uniform answer).
template <int NPER>
__device__ __forceinline__ bool slots_ready(const RowSlots<NPER>& q, int C, uint32_t tag, int lane) {
  bool ok = true;
#pragma unroll
  for (int j = 0; j < NPER; ++j)
    if (lane + 64 * j < C) {
#pragma unroll
      for (int k = 0; k < kX1; ++k) ok &= slot_tag(q.w[j][k]) == tag;
    }
  return __all(ok);
}
// The partials of row r (one 16-byte load per chunk, sc1 as the slots).
template <int NPER>
__device__ __forceinline__ void part_issue(const Params& P, int r, bool real, const uint32_t (&off)[NPER],
                                           float4 (&pt)[NPER]) {
  const Rsrc rs = __builtin_amdgcn_make_buffer_rsrc((void*)(P.part + (int64_t)(real ? r : 0) * P.C * kPart),
                                                    (short)0, real ? P.C * kPart * (int)sizeof(float) : 0,
                                                    kRsrcWord3);
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off[j], 0, kSC1);
    pt[j] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
  }
}
template <int NPER>
__device__ __forceinline__ bool parts_ready(const float4 (&pt)[NPER], int C, uint32_t tag, int lane) {
  bool ok = true;
#pragma unroll
  for (int j = 0; j < NPER; ++j)
    if (lane + 64 * j < C) ok &= __float_as_uint(pt[j].x) == tag;
  return __all(ok);
}
// Row normalisers of a softmax split into chunks from slots (m_c, s_c) at
// slot index `at`: M = max m_c, S = sum s_c 2^((m_c - M) s).  Every caller
// uses the same lane layout, so every wave gets the same bits.
template <int NPER>
__device__ __forceinline__ void merge_row(const RowSlots<NPER>& q, int C, int at, float s, int lane, float& M,
                                          float& S) {
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int j = 0; j < NPER; ++j)
    if (lane + 64 * j < C) m = fmaxf(m, slot_f(q.w[j][at]));
  M = wave_max(m);
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < NPER; ++j)
    if (lane + 64 * j < C) a += slot_f(q.w[j][at + 1]) * __builtin_amdgcn_exp2f(chunk_exp(slot_f(q.w[j][at]), M, s));
  S = wave_sum(a);
}
__device__ __forceinline__ bool norm_ok(float M, float S) {
  return M > -__builtin_huge_valf() && S == S && S > 0.0f && S <= kFltMax;
}

// ------------------------------------------------------------------ loads

// A raw buffer over chunk c of a row: bytes c * kRowBytes .. nb of the row.
// Every load through it uses a vector offset relative to the chunk start,
// which the hardware checks against the buffer's size, so bytes past the
// row end read as 0 and no load leaves the row.  live false: a zero-sized
// buffer (every load reads 0 and touches no memory).
__device__ __forceinline__ Rsrc chunk_rsrc(const char* base, int row, uint32_t stride_b, int c, int nb,
                                           bool live) {
  // the address is formed whatever `live` is: a zero-sized buffer never touches memory
  const char* p = base + (uint64_t)(uint32_t)row * stride_b + (uint32_t)(c * kRowBytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, live ? nb - c * kRowBytes : 0, kRsrcWord3);
}

// Load u of one row of a chunk: lane `lane` gets tokens u*64*EPV +
// lane*EPV .. +EPV-1 of the chunk.  VEC: one 16-byte load (rows and V*esize
// on 16-byte boundaries); otherwise element loads.
template <int DT, bool VEC>
__device__ __forceinline__ u32x4 load_vec(Rsrc rs, int u, int lane) {
  using F = Fmt<DT>;
  u32x4 w;
  if (VEC) {
    w = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + u * 1024, 0, kNT);
  } else {
    const int t0 = u * 64 * F::EPV + lane * F::EPV;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (DT == SPECVERIFY_F32) {
        w[e] = __builtin_amdgcn_raw_buffer_load_b32(rs, (t0 + e) * 4, 0, kNT);
      } else {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, (t0 + 2 * e) * 2, 0, kNT);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, (t0 + 2 * e + 1) * 2, 0, kNT);
        w[e] = lo | (hi << 16);
      }
    }
  }
  return w;
}
template <int DT, bool VEC>
__device__ __forceinline__ void issue_row(Rsrc rs, int lane, u32x4 (&raw)[kU]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) raw[u] = load_vec<DT, VEC>(rs, u, lane);
}

template <int DT>
__device__ __forceinline__ void unpack(const u32x4 (&raw)[kU], float (&x)[Fmt<DT>::L]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = raw[u][e];
      if (DT == SPECVERIFY_F32) {
        x[u * 4 + e] = __uint_as_float(w);
      } else {
        x[u * 8 + 2 * e] = __uint_as_float(w << 16);
        x[u * 8 + 2 * e + 1] = __uint_as_float(w & 0xFFFF0000u);
      }
    }
  }
}
// Tokens >= V of the last chunk become -inf, in two rows of the same chunk
// at once: one comparison per token, and one at a time (each comparison's
// lane mask is used at once), which keeps the scalar registers of this rare
// path from crowding the common one.
// TWO false: only x is masked (y may alias it).
template <int DT, bool TWO = true>
__device__ __forceinline__ void mask_tail2(float (&x)[Fmt<DT>::L], float (&y)[Fmt<DT>::L], int c, int V, int lane) {
  using F = Fmt<DT>;
  const int lim = V - (c * F::CH + lane * F::EPV);
#pragma unroll
  for (int u = 0; u < kU; ++u)
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) {
      const bool out = u * 64 * F::EPV + e >= lim;
      x[u * F::EPV + e] = out ? -__builtin_huge_valf() : x[u * F::EPV + e];
      if (TWO) y[u * F::EPV + e] = out ? -__builtin_huge_valf() : y[u * F::EPV + e];
      __builtin_amdgcn_sched_barrier(0);
    }
}
// Token of element k = u * EPV + e of a lane in chunk c.
template <int DT>
__device__ __forceinline__ int token_of(int c, int k, int lane) {
  using F = Fmt<DT>;
  const int u = k / F::EPV, e = k - u * F::EPV;
  return c * F::CH + u * 64 * F::EPV + lane * F::EPV + e;
}
// Element e of a lane's 16-byte vector w, as unpack leaves it.
template <int DT>
__device__ __forceinline__ float vec_elem(const u32x4& w, int e) {
  if (DT == SPECVERIFY_F32) return __uint_as_float(w[e]);
  const uint32_t h = w[e >> 1];
  return __uint_as_float((e & 1) ? (h & 0xFFFF0000u) : (h << 16));
}
// The same, with tokens >= V as -inf; `lim` is V minus the token of element
// 0 of the vector.
template <int DT>
__device__ __forceinline__ float elem(const u32x4& w, int e, int lim) {
  return e >= lim ? -__builtin_huge_valf() : vec_elem<DT>(w, e);
}
// Tokens >= V of the last chunk become -inf in the raw words of a row (one
// comparison per token, as in mask_tail2).
template <int DT>
__device__ __forceinline__ void mask_raw(u32x4 (&raw)[kU], int c, int V, int lane) {
  using F = Fmt<DT>;
  const int lim = V - (c * F::CH + lane * F::EPV);
#pragma unroll
  for (int u = 0; u < kU; ++u)
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) {
      const bool out = u * 64 * F::EPV + e >= lim;
      if (DT == SPECVERIFY_F32) {
        raw[u][e] = out ? 0xFF800000u : raw[u][e];
      } else {
        const uint32_t w = raw[u][e >> 1];
        const uint32_t m = (e & 1) ? ((w & 0x0000FFFFu) | 0xFF800000u) : ((w & 0xFFFF0000u) | 0x0000FF80u);
        raw[u][e >> 1] = out ? m : w;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// ------------------------------------------------------------------ sequence layout

// Read-only inputs that a wave reads at a uniform address go through the
// constant address space, so they become scalar loads (counted apart from
// the vector loads that the pipeline keeps in flight).
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// Unsigned division of n by a run-time constant d with the constants
// {m, s1, s2} of Granlund and Montgomery ("Division by Invariant Integers
// using Multiplication", 1994, unsigned case): l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1, s1 = min(l, 1), s2 = max(l - 1, 0);
// then t = mulhi(m, n) and n / d = (t + ((n - t) >> s1)) >> s2 for every
// 32-bit n.  Wave-uniform operands make this a few scalar instructions.
__device__ __forceinline__ uint32_t udiv(uint32_t n, const uint32_t (&k)[3]) {
  const uint32_t t = __umulhi(k[0], n);
  return (t + ((n - t) >> k[1])) >> k[2];
}

__device__ __forceinline__ bool t_sampled(float T) { return T >= kFltMin && T <= kFltMax; }
__device__ __forceinline__ bool u_ok(float u) { return u >= 0.0f && u < 1.0f; }   // false for NaN

// Rows [r0, r1) and sequences [s0, s1) of row group g.
struct Group {
  int r0, r1, s0, s1;
};
__device__ __forceinline__ Group group_of(const Params& P, int g) {
  Group G;
  if (P.gbounds == nullptr) {
    G.r0 = P.grow[g];
    G.r1 = P.grow[g + 1];
    G.s0 = P.gseq[g];
    G.s1 = P.gseq[g + 1];
  } else {
    G.r0 = ld_const(P.gbounds, g);
    G.r1 = ld_const(P.gbounds, g + 1);
    G.s0 = ld_const(P.gbounds, kGroups + 1 + g);
    G.s1 = ld_const(P.gbounds, kGroups + 2 + g);
  }
  return G;
}

// ================================================================== layout kernel (ragged batches)

// One workgroup: checks that cu_draft is a layout (cu_draft[0] = 0,
// cu_draft[B] = R_d, 0 <= gamma_b <= max_gamma); writes every target row's
// record and splits the batch into kGroups ranges of whole sequences with
// about R_t / kGroups target rows each (group g starts at the first
// sequence b whose first target row cu_draft[b] + b is at least
// g R_t / kGroups).  An invalid layout makes every group empty.
__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(Params P, int4* rowinfo, int32_t* gbounds,
                                                                uint32_t* flag) {
  const int tid = threadIdx.x;
  int bad = 0;
  for (int b = tid; b < P.B; b += blockDim.x) {
    const int g = P.cu_draft[b + 1] - P.cu_draft[b];
    bad |= g < 0 || g > P.max_gamma;
  }
  if (tid == 0) bad |= P.cu_draft[0] != 0 || P.cu_draft[P.B] != P.R_d;
  bad = __syncthreads_or(bad);
  if (bad) {
    if (tid < 2 * (kGroups + 1)) gbounds[tid] = 0;
  } else {
    for (int b = tid; b < P.B; b += blockDim.x) {
      const int d0 = P.cu_draft[b], g = P.cu_draft[b + 1] - d0;
      const int Tb = __float_as_int(P.temps[b]);
      // a tree's rows have no draft to test in the streaming pass
      for (int i = 0; i <= g; ++i) rowinfo[d0 + b + i] = make_int4(b, d0 + i, (i < g && !P.tree) ? 1 : 0, Tb);
    }
    if (tid <= kGroups) {
      // first sequence whose first target row reaches tid * R_t / kGroups
      const int64_t want = ((int64_t)tid * P.R_t + kGroups - 1) / kGroups;
      int lo = 0, hi = P.B;   // answer in [lo, hi]
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)P.cu_draft[mid] + mid >= want) hi = mid;
        else lo = mid + 1;
      }
      gbounds[tid] = P.cu_draft[lo] + lo;            // first target row of the group
      gbounds[kGroups + 1 + tid] = lo;               // first sequence of the group
    }
  }
  if (tid == 0) *flag = P.epoch * 2u + (bad ? 1u : 0u);
}

// ================================================================== streaming pass

// An item in three scalar registers: target row (bits 0-23) and chunk (bits
// 24-31); draft row (bits 0-23), mode (bits 24-25: 0 nothing to do,
// 1 sampled, 2 greedy), whether the launch reads the position's draft
// logits (bit 26), whether the position has a drafted token (bit 27) and
// whether the item exists (bit 28); log2(e) / T.  Rows < 2^24 and chunks
// <= 256 fit.  An item's loads depend only on its rows and chunk, not on
// the temperature, so that they can go out before T has been read.
struct Item {
  uint32_t rc, rdf;
  float s;
  __device__ __forceinline__ int r() const { return (int)(rc & 0xFFFFFFu); }
  __device__ __forceinline__ int c() const { return (int)(rc >> 24); }
  __device__ __forceinline__ int rd() const { return (int)(rdf & 0xFFFFFFu); }
  __device__ __forceinline__ int mode() const { return (int)((rdf >> 24) & 3u); }
  __device__ __forceinline__ bool pair() const { return (rdf >> 26) & 1u; }   // draft logits read
  __device__ __forceinline__ bool drafted() const { return (rdf >> 27) & 1u; }
  __device__ __forceinline__ bool exists() const { return (rdf >> 28) & 1u; }
};

// Item `idx` of the row-major item list of a group whose rows start at r0:
// its rows, chunk and flags, everything its loads need (mode and s are
// filled in by item_mode, which reads the temperature).
__device__ __forceinline__ Item make_item(const Params& P, int r0, int idx, int n_items) {
  Item it;
  it.rc = 0;
  it.rdf = 0;
  it.s = 0.0f;
  if (idx >= n_items) return it;
  const int rl = (int)udiv((uint32_t)idx, P.div_c);
  const int c = idx - rl * P.C;
  const int r = r0 + rl;
  it.rc = (uint32_t)r | ((uint32_t)c << 24);
  int rd, pair;
  if (P.rowinfo == nullptr) {
    const int b = (int)udiv((uint32_t)r, P.div_g);
    const int i = r - b * (P.gamma + 1);
    pair = i < P.gamma;
    rd = b * P.gamma + i;
  } else {
    const int* info = (const int*)(P.rowinfo + r);
    rd = ld_const(info, 1);
    pair = ld_const(info, 2);
  }
  // a token-only draft has no logits: its position streams like one without a draft
  it.rdf = (uint32_t)rd | ((uint32_t)(pair != 0 && !P.token_only) << 26) | ((uint32_t)(pair != 0) << 27) |
           (1u << 28);
  return it;
}
// The item's mode (bits 24-25 of rdf) and s = log2(e) / T from its
// sequence's temperature; any temperature that is neither 0 nor a usable
// positive value is invalid data: mode 0, nothing is computed.
__device__ __forceinline__ void item_mode(const Params& P, Item& it) {
  if (!it.exists()) return;
  const int r = it.r();
  const float T = P.rowinfo == nullptr ? ld_const(P.temps, (int)udiv((uint32_t)r, P.div_g))
                                       : __int_as_float(ld_const((const int*)(P.rowinfo + r), 3));
  uint32_t mode = 0;
  if (t_sampled(T)) {
    mode = 1;
    it.s = kLog2e / T;
  } else if (T == 0.0f) {
    mode = 2;
  }
  it.rdf |= mode << 24;
}

// The item's loads: always the same 2 kU (VEC) instructions; absent rows
// read through zero-sized buffers.  Element loads (rows not on 16-byte
// boundaries, a rare layout) are not prefetched: phase 1 issues them itself
// (NOW), which keeps the many element loads of a prefetch out of the
// registers of the pipeline.
template <int DT, bool VEC, bool NOW = false>
__device__ __forceinline__ void issue_item(const Params& P, const Item& it, int lane, u32x4 (&R)[2][kU]) {
  if (!VEC && !NOW) return;
  const int nb = P.V * Fmt<DT>::ESIZE;
  const bool live = it.exists();   // an invalid temperature reads what it never uses
  issue_row<DT, VEC>(chunk_rsrc(P.target, it.r(), P.tstride_b, it.c(), nb, live), lane, R[0]);
  issue_row<DT, VEC>(chunk_rsrc(P.draft, it.rd(), P.dstride_b, it.c(), nb, live && it.pair()), lane, R[1]);
}
template <int DT, bool VEC, bool NOW = false>
__device__ __forceinline__ void issue_target(const Params& P, const Item& it, int lane, u32x4 (&R)[kU]) {
  if (!VEC && !NOW) return;
  issue_row<DT, VEC>(chunk_rsrc(P.target, it.r(), P.tstride_b, it.c(), P.V * Fmt<DT>::ESIZE, it.exists()),
                     lane, R);
}

// Phase 1 of a sampled row: chunk max, exponentials in place, chunk sum.
template <int DT>
__device__ __forceinline__ void p1_row(float (&x)[Fmt<DT>::L], float s, float& m, float& sum) {
  float mm = -__builtin_huge_valf();
#pragma unroll
  for (int k = 0; k < Fmt<DT>::L; ++k) mm = fmaxf(mm, x[k]);
  m = wave_max(mm);
  const float c = chunk_offset(m, s);
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < Fmt<DT>::L; ++k) {
    x[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[k], s, c));
    a += x[k];
  }
  sum = wave_sum(a);
}

// Chunk argmax of a greedy row (first maximum in token order) and a flag for
// NaN / +inf.
template <int DT>
__device__ __forceinline__ void greedy_row(const float (&x)[Fmt<DT>::L], int c, int lane, float& v, int& k,
                                           int& bad) {
  float bv = -__builtin_huge_valf();
  int slot = -1, b = 0;
#pragma unroll
  for (int j = 0; j < Fmt<DT>::L; ++j) {
    const float y = x[j];
    b |= (y != y) | (y == __builtin_huge_valf());
    if (y > bv) {
      bv = y;
      slot = j;
    }
  }
  int bk = slot < 0 ? 0x7FFFFFFF : token_of<DT>(c, slot, lane);
  wave_argmax(bv, bk);
  v = bv;
  k = bk;
  bad = __any(b);
}

// Phase 1 of an item; publishes the chunk statistics.  `mt`, `md` keep the
// chunk maxima for phase 2.
// Both rows are unpacked whatever the item is, so that on every path the
// compiler sees the item's loads consumed here and never waits for them
// later (rows that were not read hold zeros).  Likewise every path ends in
// the same one store (items with nothing to publish write the dummy slots),
// so the count of memory operations in flight is the same on all paths.
// D false: the launch has no draft logits; only row 0 exists.  `x` (D
// false, sampled rows): a drafted token; if this chunk holds it, slot 2
// carries e_t at x instead of the absent draft's maximum.
// Once the item is unpacked, `mid` runs (the caller's memory operations that
// must go out before the next item's loads), then the loads of `next` go
// into R, which the unpack freed.
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};
template <typename H> struct IsNoHook { static constexpr bool value = false; };
template <> struct IsNoHook<NoHook> { static constexpr bool value = true; };
template <int DT, bool VEC, bool D = true, typename Hook = NoHook>
__device__ __forceinline__ void p1_item(const Params& P, const Item& it, int lane, uint64_t* wdummy,
                                        u32x4 (&R)[2][kU], float (&E)[2][Fmt<DT>::L], float& mt,
                                        float& md, float& st, int x = -1, const Item* next = nullptr,
                                        Hook mid = Hook()) {
  if (!VEC) {   // element loads: issued here, not prefetched
    if (D) issue_item<DT, VEC, true>(P, it, lane, R);
    else issue_target<DT, VEC, true>(P, it, lane, R[0]);
  }
  unpack<DT>(R[0], E[0]);
  if (D) unpack<DT>(R[1], E[1]);
  if constexpr (!IsNoHook<Hook>::value) {
    __builtin_amdgcn_sched_barrier(0);
    mid();
  }
  if (next != nullptr) {   // R is free: the next item's loads go out now
    __builtin_amdgcn_sched_barrier(0);
    issue_item<DT, VEC>(P, *next, lane, R);
    __builtin_amdgcn_sched_barrier(0);
  }
  uint32_t v0 = 0, v1 = 0, v2 = 0, v3 = 0;
  uint64_t* dst = wdummy;
  if (it.mode() != 0) {
    dst = P.xch1 + ((int64_t)it.r() * P.C + it.c()) * kX1;
    if ((it.c() + 1) * Fmt<DT>::CH > P.V) mask_tail2<DT, D>(E[0], E[1], it.c(), P.V, lane);
    if (it.mode() == 1) {
      float sd = 0.0f;
      md = -__builtin_huge_valf();
      p1_row<DT>(E[0], it.s, mt, st);
      if (D && it.pair()) p1_row<DT>(E[1], it.s, md, sd);
      v0 = __float_as_uint(mt);
      v1 = __float_as_uint(st);
      v2 = __float_as_uint(md);
      v3 = __float_as_uint(sd);
      const int t = x - it.c() * Fmt<DT>::CH;   // x's position in the chunk
      if (!D && x >= 0 && x < P.V && t >= 0 && t < Fmt<DT>::CH) {
        using F = Fmt<DT>;
        const int k = (t / (64 * F::EPV)) * F::EPV + t % F::EPV;   // element of lane (t / EPV) % 64
        float ex = 0.0f;
#pragma unroll
        for (int i = 0; i < F::L; ++i) ex = i == k ? E[0][i] : ex;
        v2 = __float_as_uint(lane_f(ex, (t / F::EPV) & 63));
      }
    } else {
      float vt, vd = -__builtin_huge_valf();
      int kt, kd = 0x7FFFFFFF, bt, bd = 0;
      greedy_row<DT>(E[0], it.c(), lane, vt, kt, bt);
      if (D && it.pair()) greedy_row<DT>(E[1], it.c(), lane, vd, kd, bd);
      v0 = __float_as_uint(vt);
      v1 = bt ? 0xFFFFFFFFu : (uint32_t)kt;
      v2 = __float_as_uint(vd);
      v3 = bd ? 0xFFFFFFFFu : (uint32_t)kd;
    }
  }
  uint32_t v = lane == 2 ? v2 : v3;   // selects, not a chain of branches on the lane
  v = lane == 1 ? v1 : v;
  v = lane == 0 ? v0 : v;
  if (lane < kX1) slot_put(dst + lane, P.epoch, v);
}

// ------------------------------------------------------------------ recomputation from memory (help)
// What phase 1 and phase 2 compute for one chunk, read again from memory one
// vector at a time (few registers; a rare path): the same operations on the
// same values in the same order, hence the same bits.

template <int DT, bool VEC>
__device__ __forceinline__ void stats_mem(Rsrc rs, int c, int V, int lane, float s, float& m, float& sum) {
  using F = Fmt<DT>;
  const int lim0 = V - (c * F::CH + lane * F::EPV);
  float mm = -__builtin_huge_valf();
#pragma unroll 1
  for (int u = 0; u < kU; ++u) {
    const u32x4 w = load_vec<DT, VEC>(rs, u, lane);
    const int lim = lim0 - u * 64 * F::EPV;
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) mm = fmaxf(mm, elem<DT>(w, e, lim));
  }
  m = wave_max(mm);
  const float off = chunk_offset(m, s);
  float a = 0.0f;
#pragma unroll 1
  for (int u = 0; u < kU; ++u) {
    const u32x4 w = load_vec<DT, VEC>(rs, u, lane);
    const int lim = lim0 - u * 64 * F::EPV;
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) a += __builtin_amdgcn_exp2f(__builtin_fmaf(elem<DT>(w, e, lim), s, off));
  }
  sum = wave_sum(a);
}
template <int DT, bool VEC>
__device__ __forceinline__ void greedy_mem(Rsrc rs, int c, int V, int lane, float& v, int& k, int& bad) {
  using F = Fmt<DT>;
  const int lim0 = V - (c * F::CH + lane * F::EPV);
  float bv = -__builtin_huge_valf();
  int slot = -1, b = 0;
#pragma unroll 1
  for (int u = 0; u < kU; ++u) {
    const u32x4 w = load_vec<DT, VEC>(rs, u, lane);
    const int lim = lim0 - u * 64 * F::EPV;
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) {
      const float y = elem<DT>(w, e, lim);
      b |= (y != y) | (y == __builtin_huge_valf());
      const bool up = y > bv;
      bv = up ? y : bv;
      slot = up ? u * F::EPV + e : slot;
    }
  }
  int bk = slot < 0 ? 0x7FFFFFFF : token_of<DT>(c, slot, lane);
  wave_argmax(bv, bk);
  v = bv;
  k = bk;
  bad = __any(b);
}
// Phase 1's four slot values of chunk c of row r (see p1_item).
template <int DT, bool VEC, bool D>
__device__ __forceinline__ void slots_mem(const Params& P, int r, int rd, int mode, bool dlog, bool drafted, float s,
                                          int c, int lane, uint32_t (&v)[kX1]) {
  const int nb = P.V * Fmt<DT>::ESIZE;
  const Rsrc rt = chunk_rsrc(P.target, r, P.tstride_b, c, nb, true);
  const Rsrc rdr = chunk_rsrc(P.draft, rd, P.dstride_b, c, nb, dlog);
  if (mode == 1) {
    float mt, st, md = -__builtin_huge_valf(), sd = 0.0f;
    stats_mem<DT, VEC>(rt, c, P.V, lane, s, mt, st);
    if (D && dlog) stats_mem<DT, VEC>(rdr, c, P.V, lane, s, md, sd);
    v[0] = __float_as_uint(mt);
    v[1] = __float_as_uint(st);
    v[2] = __float_as_uint(md);
    v[3] = __float_as_uint(sd);
    if (!D && drafted) {
      const int x = ld_const(P.tokens, rd);
      if (x >= 0 && x < P.V && x / Fmt<DT>::CH == c) {
        float lx;
        const char* row = P.target + (uint64_t)(uint32_t)r * P.tstride_b;
        if (DT == SPECVERIFY_F32) lx = ld_const((const float*)row, x);
        else lx = __uint_as_float((uint32_t)ld_const((const uint16_t*)row, x) << 16);
        v[2] = __float_as_uint(__builtin_amdgcn_exp2f(__builtin_fmaf(lx, s, chunk_offset(mt, s))));
      }
    }
  } else {
    float vt, vd = -__builtin_huge_valf();
    int kt, kd = 0x7FFFFFFF, bt, bd = 0;
    greedy_mem<DT, VEC>(rt, c, P.V, lane, vt, kt, bt);
    if (D && dlog) greedy_mem<DT, VEC>(rdr, c, P.V, lane, vd, kd, bd);
    v[0] = __float_as_uint(vt);
    v[1] = bt ? 0xFFFFFFFFu : (uint32_t)kt;
    v[2] = __float_as_uint(vd);
    v[3] = bd ? 0xFFFFFFFFu : (uint32_t)kd;
  }
}
// A wave that has polled long enough for the slots of row r computes the
// missing chunks' statistics itself (their owners may not even be running:
// nothing guarantees that every workgroup of the grid is resident at once)
// and publishes them; the owners later write the same bits.  The caller
// polls again afterwards.
template <int DT, bool VEC, bool D, int NPER>
__device__ __forceinline__ void help_slots(const Params& P, int r, int rd, int mode, bool dlog, bool drafted, float s,
                                        int lane, const RowSlots<NPER>& q) {
  const uint32_t tag = P.epoch;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    bool m = false;
    if (lane + 64 * j < P.C) {
#pragma unroll
      for (int k = 0; k < kX1; ++k) m |= slot_tag(q.w[j][k]) != tag;
    }
    uint64_t mask = __ballot(m);
    while (mask) {
      const int c = __builtin_ctzll(mask) + 64 * j;
      mask &= mask - 1;
      uint32_t v[kX1];
      slots_mem<DT, VEC, D>(P, r, rd, mode, dlog, drafted, s, c, lane, v);
      uint32_t y = lane == 2 ? v[2] : v[3];
      y = lane == 1 ? v[1] : y;
      y = lane == 0 ? v[0] : y;
      if (lane < kX1) slot_put(P.xch1 + ((int64_t)r * P.C + c) * kX1 + lane, tag, y);
    }
  }
}
// The same for missing partials of a sampled row with draft logits, once its
// slots are complete (in q): phase 2 of each missing chunk from memory.
template <int DT, bool VEC, int NPER>
__device__ __forceinline__ void help_parts(const Params& P, int r, int rd, float s, int lane, const RowSlots<NPER>& q,
                                        const float4 (&pt)[NPER]) {
  using F = Fmt<DT>;
  const uint32_t tag = P.epoch;
  float Mt, St, Md, Sd;
  merge_row(q, P.C, 0, s, lane, Mt, St);
  merge_row(q, P.C, 2, s, lane, Md, Sd);
  const int nb = P.V * F::ESIZE;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    uint64_t mask = __ballot(lane + 64 * j < P.C && __float_as_uint(pt[j].x) != tag);
    while (mask) {
      const int l = __builtin_ctzll(mask);
      const int c = l + 64 * j;
      mask &= mask - 1;
      const float mt = __int_as_float(__builtin_amdgcn_readlane((int)(uint32_t)q.w[j][0], l));
      const float st = __int_as_float(__builtin_amdgcn_readlane((int)(uint32_t)q.w[j][1], l));
      const float md = __int_as_float(__builtin_amdgcn_readlane((int)(uint32_t)q.w[j][2], l));
      const float rho = chunk_rho(mt, Mt, St, md, Md, Sd, s);
      const float ct = chunk_offset(mt, s), cd = chunk_offset(md, s);
      const Rsrc rt = chunk_rsrc(P.target, r, P.tstride_b, c, nb, true);
      const Rsrc rdr = chunk_rsrc(P.draft, rd, P.dstride_b, c, nb, true);
      const int lim0 = P.V - (c * F::CH + lane * F::EPV);
      float b = 0.0f;
#pragma unroll 1
      for (int u = 0; u < kU; ++u) {
        const u32x4 wt = load_vec<DT, VEC>(rt, u, lane);
        const u32x4 wd = load_vec<DT, VEC>(rdr, u, lane);
        const int lim = lim0 - u * 64 * F::EPV;
#pragma unroll
        for (int e = 0; e < F::EPV; ++e) {
          const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(elem<DT>(wt, e, lim), s, ct));
          const float ed = __builtin_amdgcn_exp2f(__builtin_fmaf(elem<DT>(wd, e, lim), s, cd));
          b += min_nonneg(et, rho * ed);
        }
      }
      const float bs = wave_sum(b);
      if (lane == 0)
        *(float4*)(P.part + ((int64_t)r * P.C + c) * kPart) =
            make_float4(__uint_as_float(tag), fmaxf(st - bs, 0.0f), bs, 0.0f);
    }
  }
}

// Phase 2 of a sampled item with a draft, once its row's slots are in `q`
// (`ready`: they all carry this run's tag).  Leaves the partials in `o` and
// their address in `dst`; the caller stores them.
template <int DT, bool VEC, int NPER, bool HX>
__device__ __forceinline__ void p2_item(const Params& P, const Item& it, int lane, const uint32_t (&soff)[NPER],
                                        RowSlots<NPER>& q, bool ready, const float (&Et)[Fmt<DT>::L],
                                        const float4* sxt, const float4* sed, float mt, float md, float st,
                                        float4& o, float*& dst) {
  const uint32_t tag = P.epoch;
  if (!ready) {
    for (int k = 0;; ++k) {
      // the help makes the next poll succeed; the bound only guards that
      if (k > 2 * P.spin_limit + 16) return;   // no partials: the resolution reports it
      if (k == P.spin_limit) {
        help_slots<DT, VEC, true, NPER>(P, it.r(), it.rd(), 1, true, true, it.s, lane, q);
        __builtin_amdgcn_s_waitcnt(0);   // its stores are in L2 before the poll below
      } else {
        __builtin_amdgcn_s_sleep(2);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the loads below are read again on every turn
      slots_issue(P, it.r(), true, soff, q);
      if (slots_ready(q, P.C, tag, lane)) break;
    }
  }
  float Mt, St, Md, Sd;
  merge_row(q, P.C, 0, it.s, lane, Mt, St);
  merge_row(q, P.C, 2, it.s, lane, Md, Sd);
  // invalid data gives NaN or inf here; the resolution checks the normalisers
  const float rho = chunk_rho(mt, Mt, St, md, Md, Sd, it.s);   // q_k = a_t rho e_d
  // sum of min(e_t, rho e_d); the residual's sum is the chunk sum of e_t
  // (phase 1's st, the same values added in the same order) minus it
  float b = 0.0f;
#pragma unroll
  for (int k4 = 0; k4 < Fmt<DT>::L / 4; ++k4) {
    const float4 d = sed[k4 * 64 + lane];
    const bool lo = HX && k4 < Fmt<DT>::L / 8;
    const float4 t = lo ? sxt[k4 * 64 + lane]
                        : make_float4(Et[4 * k4], Et[4 * k4 + 1], Et[4 * k4 + 2], Et[4 * k4 + 3]);
    b += min_nonneg(t.x, rho * d.x);
    b += min_nonneg(t.y, rho * d.y);
    b += min_nonneg(t.z, rho * d.z);
    b += min_nonneg(t.w, rho * d.w);
  }
  const float bs = wave_sum(b);
  o.x = __uint_as_float(tag);
  o.y = fmaxf(st - bs, 0.0f);
  o.z = bs;
  dst = P.part + ((int64_t)it.r() * P.C + it.c()) * kPart;
}

// The exponentials an item keeps for its phase 2 in the wave's LDS area:
// e_d, and with HX the lower half of e_t (the rest of e_t stays in
// registers).  HX is taken where the chunk slots of a row need more than
// one register set per lane (NPER > 1): there the registers would not leave
// room for three waves per SIMD.
template <int NPER>
constexpr bool kHalfInLds = NPER > 1;
template <int DT, bool HX>
__device__ __forceinline__ void keep_item(const float (&E)[2][Fmt<DT>::L], int lane, float4* sxt, float4* sed) {
#pragma unroll
  for (int k4 = 0; k4 < Fmt<DT>::L / 4; ++k4) {
    sed[k4 * 64 + lane] = make_float4(E[1][4 * k4], E[1][4 * k4 + 1], E[1][4 * k4 + 2], E[1][4 * k4 + 3]);
    if (HX && k4 < Fmt<DT>::L / 8)
      sxt[k4 * 64 + lane] = make_float4(E[0][4 * k4], E[0][4 * k4 + 1], E[0][4 * k4 + 2], E[0][4 * k4 + 3]);
  }
}

// One pipeline step of a wave (launches with draft logits):
//   phase 1 of n1, whose loads were issued a step ago; once it is unpacked,
//   the poll of cur's row goes out, then the loads of n2 into the freed
//   buffer; then the wait for the poll and phase 2 of cur (its e_t, or its
//   upper half, in Ecur, the rest of its exponentials in the wave's LDS
//   area), and n1's exponentials replace cur's there.
// Vector memory operations complete in order: the poll, issued before n2's
// loads, waits only for what phase 1 of n1 has consumed already.  cur's own
// phase 1 ran a whole step earlier, so the other chunks of its row have
// mostly published by the time the poll reads them.
// A wave holds one item's loads and at most one and a half items'
// exponentials in registers, which leaves room for three waves per SIMD.
// Every path through a step issues the same memory operations (items that
// do not exist read zero-sized buffers and write the dummy slots), so the
// compiler's count of operations in flight is exact at every wait.
template <int DT, bool VEC, int NPER>
__device__ __forceinline__ void step(const Params& P, int lane, uint64_t* wdummy, const uint32_t (&soff)[NPER],
                                     RowSlots<NPER>& q, const Item& cur, const float (&Ecur)[Fmt<DT>::L],
                                     float4* sxt, float4* sed, float cmt, float cmd, float cst, const Item& n1,
                                     u32x4 (&R)[2][kU], float (&Efree)[2][Fmt<DT>::L], float& nmt, float& nmd,
                                     float& nst, const Item& n2, bool& behind) {
  // Phase 1 publishes what other waves' phase 2 polls for: it runs at a
  // raised issue priority, the highest for a wave that was behind the other
  // waves of its last row (that row was complete at its first poll).
  if (behind) {
    __builtin_amdgcn_s_setprio(3);
  } else {
    __builtin_amdgcn_s_setprio(1);
  }
  const bool live = cur.mode() == 1 && cur.pair();
  p1_item<DT, VEC>(P, n1, lane, wdummy, R, Efree, nmt, nmd, nst, -1, VEC ? &n2 : nullptr,
                   [&]() { slots_issue(P, cur.r(), live, soff, q); });
  __builtin_amdgcn_s_setprio(0);
  const bool ready = slots_ready(q, P.C, P.epoch, lane);   // consumes the poll on every path
  // A row complete at the first poll marks a wave that runs behind the other
  // waves of its row: the rest of its step runs at a raised priority, while a
  // wave that has to wait for its row stays at the lowest.  A step without a
  // phase 2 (an item without draft logits, or none) reads an empty buffer and
  // counts as not behind (keeping the flag across such steps measured slower).
  behind = ready;
  if (ready) __builtin_amdgcn_s_setprio(2);
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float* dst = (float*)(wdummy + kX1);
  if (live) p2_item<DT, VEC, NPER, kHalfInLds<NPER>>(P, cur, lane, soff, q, ready, Ecur, sxt, sed, cmt, cmd, cst, o, dst);
  if (lane == 0) *(float4*)dst = o;
  if (n1.mode() == 1 && n1.pair()) keep_item<DT, kHalfInLds<NPER>>(Efree, lane, sxt, sed);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

// ================================================================== resolution of a sequence

__device__ __forceinline__ uint32_t row_payload(int status, bool acc, int tok) {
  return ((uint32_t)status << kStatusShift) | (acc ? kAccBit : 0u) |
         (status == 0 ? ((uint32_t)tok & kTokMask) : 0u);
}

// a[j] for a wave-uniform j, by masks: a chain of selects can be turned
// back into an indexed load from scratch memory
template <int NPER>
__device__ __forceinline__ float pick(const float (&a)[NPER], int j) {
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) v |= __float_as_uint(a[i]) & (0u - (uint32_t)(i == j));
  return __uint_as_float(v);
}

// One logit of a row as fp32 (token t < V).
template <int DT>
__device__ __forceinline__ float load_logit(const char* base, int row, uint32_t stride_b, int t) {
  const char* p = base + (uint64_t)(uint32_t)row * stride_b;
  if (DT == SPECVERIFY_F32) return ((const float*)p)[t];
  return __uint_as_float((uint32_t)((const uint16_t*)p)[t] << 16);
}

// What a row's resolution reads: its chunk slots, its partials (rows with
// draft logits) and the drafted token.
template <int NPER>
struct RowIn {
  RowSlots<NPER> q;
  float4 pt[NPER];   // {tag, W_c, B_c} of the lane's chunks
  int x;             // drafted token (rows with a draft)
};

// The final sample of a row, prepared while the row is resolved and
// finished once the sequence's first rejection is known: the chunk whose
// CDF interval holds the threshold (its logits are re-read right away), and
// what the scan of that chunk in token order needs.
struct SampleJob {
  int row;       // row index j in the sequence; -1: none
  int cs;        // owner chunk
  float tau;     // threshold, in the chunk's units, less the mass before the chunk
  float rho, ct, cd;
  int x;         // the drafted token (removed from a token-only residual)
  bool resid;    // weights of the residual max(0, p - q); otherwise of p
  bool tk;       // token-only draft: the residual is p without x
};

// Phase A of one sampled row, on one wave, once its slots (and partials)
// are complete: p(x), q(x), beta, Z; the acceptance test u_i q(x) < p(x);
// and, for the wave's first row that needs the final sample (a rejected
// draft, or the bonus row), the owner chunk, whose logits are loaded into R.
// Returns the row result (accepted rows carry their draft token).
template <int DT, bool VEC, bool D, int NPER>
__device__ __forceinline__ uint32_t accept_sampled(const Params& P, int j, int r, int rd, bool pair, bool dp, float T,
                                                   float ui, float ug, int lane, const RowIn<NPER>& in, float lx,
                                                   float dx, SampleJob& job, u32x4 (&R)[2][kU]) {
  using F = Fmt<DT>;
  const int C = P.C;
  const float s = kLog2e / T;
  const float ninf = -__builtin_huge_valf();
  // dp: the draft's logits are there; tk: a token-only draft, q = delta_x
  const bool tk = pair && !dp;
  const int x = in.x;
  const bool x_ok = x >= 0 && x < P.V;
  const RowSlots<NPER>& q = in.q;
  float W[NPER], Bp[NPER];
#pragma unroll
  for (int jj = 0; jj < NPER; ++jj) {
    const bool inr = dp && lane + 64 * jj < C;
    W[jj] = inr ? in.pt[jj].y : 0.0f;
    Bp[jj] = inr ? in.pt[jj].z : 0.0f;
  }
  float Mt, St, Md = ninf, Sd = 0.0f;
  merge_row(q, C, 0, s, lane, Mt, St);
  if (dp) merge_row(q, C, 2, s, lane, Md, Sd);
  if (!norm_ok(Mt, St) || (dp && !norm_ok(Md, Sd)) || (pair && !x_ok)) return row_payload(1, false, 0);
  const int cx = x / F::CH;              // the chunk that holds x
  const int lxl = cx & 63, jx = cx >> 6;
  // per-chunk scales, residual mass, beta, and the masses the final sample reads
  float at[NPER], tot[NPER], mt[NPER], md[NPER], rho[NPER];
#pragma unroll
  for (int jj = 0; jj < NPER; ++jj) {
    const bool inr = lane + 64 * jj < C;
    mt[jj] = inr ? slot_f(q.w[jj][0]) : ninf;
    md[jj] = (inr && dp) ? slot_f(q.w[jj][2]) : ninf;
    at[jj] = inr ? chunk_scale(mt[jj], Mt, St, s) : 0.0f;
    rho[jj] = (inr && dp) ? chunk_rho(mt[jj], Mt, St, md[jj], Md, Sd, s) : 0.0f;
  }
  const float mtx = lane_f(pick(mt, jx), lxl);
  // e at x as phase 1 computed it (the same operations on the same values);
  // for a token-only draft phase 1 published it in slot 2 of x's chunk
  float ex;
  if (tk) {
    uint32_t vx = 0;   // slot 2 of chunk cx, read from its lane
#pragma unroll
    for (int jj = 0; jj < NPER; ++jj) {
      const uint32_t vj = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)q.w[jj][2], lxl);
      vx = jj == jx ? vj : vx;
    }
    ex = __uint_as_float(vx);
  } else {
    ex = __builtin_amdgcn_exp2f(__builtin_fmaf(lx, s, chunk_offset(mtx, s)));
  }
  if (tk) {
    // the residual p - delta_x is p without x: the chunk sums of e_t, less
    // x's own e in its chunk
#pragma unroll
    for (int jj = 0; jj < NPER; ++jj) {
      const bool inr = lane + 64 * jj < C;
      W[jj] = inr ? slot_f(q.w[jj][1]) : 0.0f;
      if (lane + 64 * jj == cx) W[jj] = fmaxf(W[jj] - ex, 0.0f);
    }
  }
  float zl = 0.0f, bl = 0.0f;
#pragma unroll
  for (int jj = 0; jj < NPER; ++jj) {
    const bool inr = lane + 64 * jj < C;
    zl += inr ? at[jj] * W[jj] : 0.0f;
    bl += inr ? at[jj] * Bp[jj] : 0.0f;
  }
  float Z = 0.0f, beta = 0.0f;
  if (pair) {
    Z = wave_sum(zl);
    beta = wave_sum(bl);
  }
  // p(x), q(x): the logits at x with their chunk's offset and scale; the
  // acceptance test u q(x) < p(x)
  if (pair) {
    const float mdx = lane_f(pick(md, jx), lxl);
    const float px = chunk_scale(mtx, Mt, St, s) * ex;
    const float qx = tk ? 1.0f : chunk_scale(mdx, Md, Sd, s) * __builtin_amdgcn_exp2f(__builtin_fmaf(dx, s, chunk_offset(mdx, s)));
    if (tk) beta = px;   // sum min(p, delta_x) = p(x)
    if (lane == 0) {
      if (P.p_draft) P.p_draft[rd] = px;
      if (P.q_draft) P.q_draft[rd] = qx;
      if (P.beta) P.beta[rd] = beta;
      if (P.resid) P.resid[rd] = Z;
    }
    if (ui * qx < px) return row_payload(0, true, x);   // an accepted draft emits itself
  }
  if (job.row >= 0) return row_payload(0, false, 0);   // an earlier row of this wave needs the sample
  // The final sample: the owner chunk is the first chunk whose cumulative
  // mass exceeds thr = u_gamma * mass (chunks with zero mass never own);
  // rounding guard: the last chunk with mass.
  const bool resid = pair && Z > 0.0f;
  float ml = 0.0f;
#pragma unroll
  for (int jj = 0; jj < NPER; ++jj) {
    const bool inr = lane + 64 * jj < C;
    tot[jj] = !inr ? 0.0f : resid ? at[jj] * W[jj] : at[jj] * slot_f(q.w[jj][1]);
    ml += tot[jj];
  }
  const float mass = resid ? Z : wave_sum(ml);
  const float thr = ug * mass;
  int cs = -1, last = -1;
  float before = 0.0f, last_before = 0.0f, base = 0.0f;
#pragma unroll
  for (int jj = 0; jj < NPER; ++jj) {
    const bool inr = lane + 64 * jj < C;
    const float t = inr ? tot[jj] : 0.0f;
    const float Gs = base + wave_scan(t, lane);
    const float Gex = Gs - t;
    const uint64_t hit = __ballot(inr && t > 0.0f && Gs > thr);
    const uint64_t pos = __ballot(inr && t > 0.0f);
    if (cs < 0 && hit) {
      const int l = __builtin_ctzll(hit);
      cs = 64 * jj + l;
      before = lane_f(Gex, l);
    }
    if (pos) {
      const int l = 63 - __builtin_clzll(pos);
      last = 64 * jj + l;
      last_before = lane_f(Gex, l);
    }
    base = lane_f(Gs, 63);
  }
  if (cs < 0) {
    cs = last;
    before = last_before;
  }
  if (cs < 0) return row_payload(2, false, 0);   // unreachable for a valid row
  const int ls = cs & 63, js = cs >> 6;
  job.row = j;
  job.cs = cs;
  job.tau = (thr - before) / lane_f(pick(at, js), ls);
  job.rho = lane_f(pick(rho, js), ls);
  job.ct = chunk_offset(lane_f(pick(mt, js), ls), s);
  job.cd = chunk_offset(lane_f(pick(md, js), ls), s);
  job.x = x;
  job.resid = resid;
  job.tk = tk;
  // re-read the owner chunk now: its loads land while the other rows resolve
  const int nb = P.V * F::ESIZE;
  issue_row<DT, VEC>(chunk_rsrc(P.target, r, P.tstride_b, cs, nb, true), lane, R[0]);
  if (D) issue_row<DT, VEC>(chunk_rsrc(P.draft, rd, P.dstride_b, cs, nb, resid && dp), lane, R[1]);
  return row_payload(0, false, 0);
}

// Phase B: the token of a prepared sample, from the re-read owner chunk in R.
// Running sums in the chunk's units against tau.  Token order inside the
// chunk is round u (one 16-byte vector per lane), then lane, then element.
// Per round: the weights (recomputed with the same functions as phase 2,
// one branch per row around straight-line code), a wave scan of the lane
// sums and the first position whose running sum exceeds tau.  Rounds go in
// order and stop at the first with a hit.  Returns the token, or -1.
template <int DT, bool D>
__device__ __forceinline__ int sample_scan(const Params& P, const SampleJob& job, float s, int lane,
                                           u32x4 (&R)[2][kU]) {
  using F = Fmt<DT>;
  const int cs = job.cs;
  if ((cs + 1) * F::CH > P.V) {   // tokens >= V: weight 0
    mask_raw<DT>(R[0], cs, P.V, lane);
    if (D) mask_raw<DT>(R[1], cs, P.V, lane);
  }
  int first = 0x7FFFFFFF, lastpos = -1;
  float rbase = 0.0f;
#pragma unroll 1
  for (int u = 0; u < kU; ++u) {
    // the round's two vectors, picked by selects (u is wave-uniform)
    u32x4 vt = R[0][0], vd = R[D ? 1 : 0][0];
#pragma unroll
    for (int i = 1; i < kU; ++i) {
      vt = i == u ? R[0][i] : vt;
      if (D) vd = i == u ? R[1][i] : vd;
    }
    float w[F::EPV];
    if (job.tk && job.resid) {
#pragma unroll
      for (int e = 0; e < F::EPV; ++e) {   // p without x
        const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(vec_elem<DT>(vt, e), s, job.ct));
        w[e] = token_of<DT>(cs, u * F::EPV + e, lane) == job.x ? 0.0f : et;
      }
    } else if (D && job.resid) {
#pragma unroll
      for (int e = 0; e < F::EPV; ++e)
        w[e] = resid_w(__builtin_amdgcn_exp2f(__builtin_fmaf(vec_elem<DT>(vt, e), s, job.ct)),
                       __builtin_amdgcn_exp2f(__builtin_fmaf(vec_elem<DT>(vd, e), s, job.cd)), job.rho);
    } else {
#pragma unroll
      for (int e = 0; e < F::EPV; ++e) w[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(vec_elem<DT>(vt, e), s, job.ct));
    }
    float loc[F::EPV];
    float run = 0.0f;
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) {
      run += w[e];
      loc[e] = run;
    }
    const float incl = wave_scan(run, lane);
    const float excl = rbase + (incl - run);
    int cand = 0x7FFFFFFF;
#pragma unroll
    for (int e = F::EPV - 1; e >= 0; --e) {
      const int k = u * 64 * F::EPV + lane * F::EPV + e;   // position inside the chunk
      if (w[e] > 0.0f) {
        if (excl + loc[e] > job.tau) cand = k;
        lastpos = max(lastpos, k);
      }
    }
    if (__ballot(cand != 0x7FFFFFFF)) {   // positions grow with the round: this round's least hit is the first
      first = wave_min_i(cand);
      break;
    }
    rbase = rbase + lane_f(incl, 63);
  }
  if (first == 0x7FFFFFFF) lastpos = wave_max_i(lastpos);   // every round was scanned
  const int pickk = first != 0x7FFFFFFF ? first : lastpos;
  const int tok = cs * F::CH + pickk;
  return (pickk < 0 || tok >= P.V) ? -1 : tok;   // unreachable: the chunk has weight > 0
}

// One row of a greedy sequence, on one wave, once its slots are complete.
template <int NPER>
__device__ __forceinline__ uint32_t finish_greedy(const Params& P, int rd, bool pair, bool dp, int lane,
                                                  const RowIn<NPER>& in) {
  const int C = P.C;
  const RowSlots<NPER>& q = in.q;
  float av = -__builtin_huge_valf(), dv = -__builtin_huge_valf();
  int ak = 0x7FFFFFFF, dk = 0x7FFFFFFF, bad = 0;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    if (lane + 64 * j < C) {
      argmax_merge(av, ak, slot_f(q.w[j][0]), (int)(uint32_t)q.w[j][1]);
      bad |= (uint32_t)q.w[j][1] == 0xFFFFFFFFu;
      if (dp) {
        argmax_merge(dv, dk, slot_f(q.w[j][2]), (int)(uint32_t)q.w[j][3]);
        bad |= (uint32_t)q.w[j][3] == 0xFFFFFFFFu;
      }
    }
  }
  bad = __any(bad);
  wave_argmax(av, ak);
  wave_argmax(dv, dk);
  if (bad || av == -__builtin_huge_valf() || (dp && dv == -__builtin_huge_valf()))
    return row_payload(1, false, 0);
  bool acc = false;
  if (pair) {
    const int x = in.x;
    if (x < 0 || x >= P.V) return row_payload(1, false, 0);
    if (!dp) dk = x;   // a token-only draft's argmax is x itself
    acc = (x == ak);
    if (lane == 0) {
      if (P.p_draft) P.p_draft[rd] = (x == ak) ? 1.0f : 0.0f;
      if (P.q_draft) P.q_draft[rd] = (x == dk) ? 1.0f : 0.0f;
      if (P.beta) P.beta[rd] = (ak == dk) ? 1.0f : 0.0f;
      if (P.resid) P.resid[rd] = (ak == dk) ? 0.0f : 1.0f;
    }
  }
  return row_payload(0, acc, ak);
}

// Row j (row r) of a sequence: wait until its slots (and, for a sampled row
// with draft logits, its partials) carry this run's tag -- computing what is
// still missing after spin_limit polls -- then resolve it (phase A).
// D: the launch has draft logits.
template <int DT, bool VEC, bool D, int NPER>
__device__ __forceinline__ uint32_t resolve_row(const Params& P, int j, int r, int rd, bool pair, float T, float ui,
                                                float ug, int lane, SampleJob& job, u32x4 (&R)[2][kU]) {
  const bool sampled = t_sampled(T);
  if (!(sampled || T == 0.0f) || !u_ok(ui)) return row_payload(1, false, 0);
  const bool dp = D && pair;                // the position's draft logits are read
  const bool dpart = dp && sampled;         // it has partials
  const float s = sampled ? kLog2e / T : 0.0f;
  uint32_t soff[NPER], poff[NPER];
  chunk_offsets(P.C, lane, kX1 * (int)sizeof(uint64_t), soff);
  chunk_offsets(P.C, lane, kPart * (int)sizeof(float), poff);
  RowIn<NPER> in;
  in.x = pair ? ld_const(P.tokens, rd) : 0;
  // the logits at x go out before the polls, so that they have landed when
  // the row's statistics have (token-only rows read e_t at x from the slots)
  float lx = 0.0f, dx = 0.0f;
  if (sampled && dp && in.x >= 0 && in.x < P.V) {
    lx = load_logit<DT>(P.target, r, P.tstride_b, in.x);
    dx = load_logit<DT>(P.draft, rd, P.dstride_b, in.x);
  }
  for (int k = 0;; ++k) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the loads below are read again on every turn
    slots_issue(P, r, true, soff, in.q);
    part_issue(P, r, dpart, poff, in.pt);
    const bool sready = slots_ready(in.q, P.C, P.epoch, lane);
    if (sready && (!dpart || parts_ready(in.pt, P.C, P.epoch, lane))) break;
    // the help makes the next poll succeed; the bound only guards that
    if (k > 2 * P.spin_limit + 16) return row_payload(2, false, 0);
    if (k == P.spin_limit) {
      if (!sready) {
        help_slots<DT, VEC, D, NPER>(P, r, rd, sampled ? 1 : 2, dp, pair, s, lane, in.q);
        __builtin_amdgcn_s_waitcnt(0);   // its stores are in L2 before the reads below
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        slots_issue(P, r, true, soff, in.q);
      }
      if (dpart && slots_ready(in.q, P.C, P.epoch, lane)) {
        help_parts<DT, VEC, NPER>(P, r, rd, s, lane, in.q, in.pt);
        __builtin_amdgcn_s_waitcnt(0);
      }
    } else {
      __builtin_amdgcn_s_sleep(2);
    }
  }
  if (sampled) return accept_sampled<DT, VEC, D, NPER>(P, j, r, rd, pair, dp, T, ui, ug, lane, in, lx, dx, job, R);
  return finish_greedy<NPER>(P, rd, pair, dp, lane, in);
}

// Sequence b, by one workgroup.  Phase A: its waves resolve the rows (row j
// on wave j mod kStreamWaves, in order), and each wave prepares the final
// sample of its first row that needs one.  The row results meet in LDS.
// Phase B: the first rejection n; the wave that holds row n (its first row
// needing the sample, since every earlier row was accepted) scans the
// re-read chunk and writes the accepted length and the n + 1 tokens.
template <int DT, bool VEC, bool D, int NPER>
__device__ __forceinline__ void resolve_sequence(const Params& P, int b, int lane, int wv, uint32_t* shres) {
  int d0, gam;
  if (P.cu_draft == nullptr) {
    d0 = b * P.gamma;
    gam = P.gamma;
  } else {
    d0 = ld_const(P.cu_draft, b);
    gam = ld_const(P.cu_draft, b + 1) - d0;
  }
  const int t0 = d0 + b;
  const float T = ld_const(P.temps, b);
  const float ug = ld_const(P.uniforms, t0 + gam);
  SampleJob job;
  job.row = -1;
  u32x4 R[2][kU];
  for (int j = wv; j <= gam; j += kStreamWaves) {
    const int r = t0 + j;
    const uint32_t res = resolve_row<DT, VEC, D, NPER>(P, j, r, d0 + j, j < gam, T, ld_const(P.uniforms, r), ug,
                                                       lane, job, R);
    if (lane == 0) shres[j] = res;
  }
  __syncthreads();
  // first rejection n and the sequence's status
  int n = gam, st = 0;
  for (int j0 = 0; j0 <= gam; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t v = j <= gam ? shres[j] : 0u;
    st = max(st, wave_max_i((int)(v >> kStatusShift)));
    const uint64_t rb = __ballot(j < gam && !(v & kAccBit));
    if (n == gam && rb) n = j0 + __builtin_ctzll(rb);
  }
  const bool sampled = t_sampled(T);
  const int writer = (st == 0 && sampled) ? n % kStreamWaves : 0;
  if (wv == writer) {
    int tn = 0;
    if (st == 0) {
      if (sampled) {
        // job.row == n here: every row of this wave before n was accepted
        tn = job.row == n ? sample_scan<DT, D>(P, job, kLog2e / T, lane, R) : -1;
        if (tn < 0) st = 2;   // unreachable
      } else {
        tn = (int)(shres[n] & kTokMask);   // greedy: the argmax
      }
    }
    // rows before n emit their drafts, row n the sampled token
    for (int j0 = 0; j0 <= gam; j0 += 64) {
      const int j = j0 + lane;
      if (j <= gam) P.out_tokens[t0 + j] = (st != 0 || j > n) ? -1 : j < n ? (int)(shres[j] & kTokMask) : tn;
    }
    if (lane == 0) P.acc_len[b] = st == 2 ? -2 : st == 1 ? -1 : n;
  }
  // the re-read of a wave whose sample was not needed lands before R is reused
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();   // shres is reused by the next sequence
}

// Every output -1: the batch layout (cu_draft) is invalid.
// tid: the thread's index in its workgroup.
__device__ __forceinline__ void invalid_batch(const Params& P, int tid) {
  const int n = P.R_t > P.B ? P.R_t : P.B;
  for (int t = blockIdx.x * blockDim.x + tid; t < n; t += gridDim.x * blockDim.x) {
    if (t < P.B) P.acc_len[t] = -1;
    if (t < P.R_t) P.out_tokens[t] = -1;
    if (t < P.R_t && P.out_nodes) P.out_nodes[t] = -1;
    if (t < P.R_d && P.p_cand) P.p_cand[t] = __builtin_nanf("");
  }
}

// ================================================================== resolution of a draft tree

// Sampling inside the owner chunk cs of a tree node's row (in R[0]): the
// first token whose cumulative weight, in the chunk's units, exceeds tau;
// the weights are the chunk's e_t, and 0 at the rejected candidates' tokens
// (nrem of them in rtok).  Token order, as sample_scan.
template <int DT>
__device__ __forceinline__ int tree_scan(const Params& P, int cs, float tau, float ct, float s, const int* rtok,
                                         int nrem, int lane, u32x4 (&R)[2][kU]) {
  using F = Fmt<DT>;
  if ((cs + 1) * F::CH > P.V) mask_raw<DT>(R[0], cs, P.V, lane);   // tokens >= V: weight 0
  int first = 0x7FFFFFFF, lastpos = -1;
  float rbase = 0.0f;
#pragma unroll 1
  for (int u = 0; u < kU; ++u) {
    u32x4 vt = R[0][0];
#pragma unroll
    for (int i = 1; i < kU; ++i) vt = i == u ? R[0][i] : vt;
    float w[F::EPV];
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) w[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(vec_elem<DT>(vt, e), s, ct));
    for (int j = 0; j < nrem; ++j) {
      const int t = rtok[j] - (cs * F::CH + u * 64 * F::EPV + lane * F::EPV);   // its element in this lane
#pragma unroll
      for (int e = 0; e < F::EPV; ++e) w[e] = t == e ? 0.0f : w[e];
    }
    float loc[F::EPV];
    float run = 0.0f;
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) {
      run += w[e];
      loc[e] = run;
    }
    const float incl = wave_scan(run, lane);
    const float excl = rbase + (incl - run);
    int cand = 0x7FFFFFFF;
#pragma unroll
    for (int e = F::EPV - 1; e >= 0; --e) {
      const int k = u * 64 * F::EPV + lane * F::EPV + e;
      if (w[e] > 0.0f) {
        if (excl + loc[e] > tau) cand = k;
        lastpos = max(lastpos, k);
      }
    }
    if (__ballot(cand != 0x7FFFFFFF)) {
      first = wave_min_i(cand);
      break;
    }
    rbase = rbase + lane_f(incl, 63);
  }
  if (first == 0x7FFFFFFF) lastpos = wave_max_i(lastpos);
  const int pickk = first != 0x7FFFFFFF ? first : lastpos;
  const int tok = cs * F::CH + pickk;
  return (pickk < 0 || tok >= P.V) ? -1 : tok;
}

// The slots of row r once all carry this run's tag (the wait ends: the help
// computes missing chunks itself).  False: the bounded wait expired.
template <int DT, bool VEC, int NPER>
__device__ __forceinline__ bool tree_poll(const Params& P, int r, int mode, float s, int lane,
                                          const uint32_t (&soff)[NPER], RowSlots<NPER>& q) {
  for (int k = 0;; ++k) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the loads below are read again on every turn
    slots_issue(P, r, true, soff, q);
    if (slots_ready(q, P.C, P.epoch, lane)) return true;
    if (k > 2 * P.spin_limit + 16) return false;
    if (k == P.spin_limit) {
      help_slots<DT, VEC, false, NPER>(P, r, 0, mode, false, false, s, lane, q);
      __builtin_amdgcn_s_waitcnt(0);   // its stores are in L2 before the poll below
    } else {
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// m of chunk cx (lane-varying) from the row's slots: slot 0 of chunk cx
// sits in lane cx mod 64 of the lane's array cx / 64.
template <int NPER>
__device__ __forceinline__ float chunk_m_of(const RowSlots<NPER>& q, int cx) {
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute((cx & 63) * 4, (int)(uint32_t)q.w[j][0]);
    v = (cx >> 6) == j ? w : v;
  }
  return __uint_as_float(v);
}

// The records of a tree's rows, in the partials area of the workspace (a
// tree launch has no phase 2): at row r, 64-bit slot 0 holds the row's
// status and, for T = 0, its argmax; slot 1 holds p of the candidate of the
// node whose row r is, under its parent's row.  Both carry the run's epoch.
__device__ __forceinline__ uint64_t* tree_rec(const Params& P, int r) {
  return (uint64_t*)(P.part + (int64_t)r * P.C * kPart);
}

// The job of one target row r of a tree, on one wave: poll the row, merge
// its normalisers (or argmax), and form the p of each of its node's
// children from the logit at its token with its chunk's offset and scale;
// write the row's record and each child's record.
template <int DT, bool VEC, int NPER>
__device__ __forceinline__ void tree_row_job(const Params& P, int r, int lane, const uint32_t (&soff)[NPER]) {
  using F = Fmt<DT>;
  const int* info = (const int*)(P.rowinfo + r);
  const int b = ld_const(info, 0);
  const float T = __int_as_float(ld_const(info, 3));
  const int n0 = ld_const(P.cu_draft, b);
  const int N = ld_const(P.cu_draft, b + 1) - n0;
  const int t0 = n0 + b;
  const int v = r - t0;   // the node whose row this is
  const bool sampled = t_sampled(T);
  const float s = sampled ? kLog2e / T : 0.0f;
  int status = 0, amax = 0;
  float M = 0.0f, S = 0.0f;
  RowSlots<NPER> q;
  if (!(sampled || T == 0.0f)) {
    status = 1;   // invalid temperature: the row was not streamed
  } else if (!tree_poll<DT, VEC, NPER>(P, r, sampled ? 1 : 2, s, lane, soff, q)) {
    status = 2;
  } else if (sampled) {
    merge_row(q, P.C, 0, s, lane, M, S);
    if (!norm_ok(M, S)) status = 1;
  } else {
    float av = -__builtin_huge_valf();
    int ak = 0x7FFFFFFF, gb = 0;
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      if (lane + 64 * j < P.C) {
        argmax_merge(av, ak, slot_f(q.w[j][0]), (int)(uint32_t)q.w[j][1]);
        gb |= (uint32_t)q.w[j][1] == 0xFFFFFFFFu;
      }
    }
    gb = __any(gb);
    wave_argmax(av, ak);
    if (gb || av == -__builtin_huge_valf()) status = 1;
    else amax = ak;
  }
  // the children: nodes k with parent v, 64 nodes per round
  for (int k0 = 1; k0 <= N; k0 += 64) {
    const int k = k0 + lane;
    const bool in = k <= N;
    const int pa = in ? P.parents[n0 + k - 1] : -1;
    const int tk = in ? P.tokens[n0 + k - 1] : -1;
    const bool child = in && pa == v;
    float p = __builtin_nanf("");
    if (status == 0) {   // wave-uniform
      if (sampled) {
        const bool ok = child && tk >= 0 && tk < P.V;
        const float l = ok ? load_logit<DT>(P.target, r, P.tstride_b, tk) : 0.0f;
        const float mx = chunk_m_of(q, ok ? tk / F::CH : 0);
        p = chunk_scale(mx, M, S, s) * __builtin_amdgcn_exp2f(__builtin_fmaf(l, s, chunk_offset(mx, s)));
      } else {
        p = tk == amax ? 1.0f : 0.0f;
      }
    }
    if (child) slot_put(tree_rec(P, t0 + k) + 1, P.epoch, __float_as_uint(p));
  }
  if (lane == 0) slot_put(tree_rec(P, r), P.epoch, ((uint32_t)status << kStatusShift) | ((uint32_t)amax & kTokMask));
}

// One sequence whose N drafts form a tree (token-only candidates), on one
// workgroup.  Perplexity "Accelerating Sonar through speculation", section
// "EAGLE" (Top-K candidates per node), with velog "6-1편. Speculative
// Decoding", sections 2-1 and 2-2 applied per candidate with q = delta_c:
// the children of the current node are tested in node order against the
// node's residual (p with the rejected candidates removed, renormalised);
// an accepted candidate is emitted and the walk moves to it; when all are
// rejected, or at a leaf, the final token is sampled from the residual by
// inverse CDF in token order.  T = 0: the child equal to the row's argmax.
//   1. nodes into LDS, checked, children lists (siblings in node order);
//   2. the four waves poll the rows (row v on wave v mod 4) and compute
//      each candidate's p under its parent's row (the logit at its token
//      with its chunk's offset and scale, as the streaming pass formed it);
//   3. wave 0 walks the tree in LDS, then samples the final token.
template <int DT, bool VEC, int NPER>
__device__ __forceinline__ void resolve_tree(const Params& P, int b, int lane, int wv) {
  using F = Fmt<DT>;
  __shared__ int tpar[kMaxGamma + 1];    // node k's parent, k >= 1
  __shared__ int ttok[kMaxGamma + 1];    // node k's candidate
  __shared__ int toff[kMaxGamma + 2];    // children of node v: tlist[toff[v] .. toff[v+1])
  __shared__ int tlist[kMaxGamma + 1];
  __shared__ float tprob[kMaxGamma + 1]; // p of node k's candidate under its parent's row
  __shared__ int tamax[kMaxGamma + 1];   // greedy: each row's argmax
  __shared__ int tpath[kMaxGamma + 1];
  __shared__ int trem[kMaxGamma + 1];    // the rejected candidates' tokens at the last node
  __shared__ float trp[kMaxGamma + 1];   // ... and the probability each removed
  __shared__ int tst;                    // worst row status
  const int tid = threadIdx.x;
  const int n0 = ld_const(P.cu_draft, b);
  const int N = ld_const(P.cu_draft, b + 1) - n0;   // in [0, max_gamma]: the layout was checked
  const int t0 = n0 + b;
  const float T = ld_const(P.temps, b);
  const bool sampled = t_sampled(T);
  const float s = sampled ? kLog2e / T : 0.0f;
  int bad = !(sampled || T == 0.0f);
  for (int k = tid + 1; k <= N; k += kStreamThreads) {
    const int pa = P.parents[n0 + k - 1], tk = P.tokens[n0 + k - 1];
    bad |= pa < 0 || pa >= k || tk < 0 || tk >= P.V;
    tpar[k] = pa;
    ttok[k] = tk;
  }
  for (int k = tid; k <= N; k += kStreamThreads) bad |= !u_ok(P.uniforms[t0 + k]);
  if (tid == 0) {
    tst = 0;
    tpar[0] = 0;
    ttok[0] = 0;
  }
  bad = __syncthreads_or(bad);
  if (!bad) {
    // children lists: node k goes to slot toff[parent] + (its rank among its siblings)
    for (int v = tid; v <= N + 1; v += kStreamThreads) {
      int o = 0;
      for (int k = 1; k <= N; ++k) o += tpar[k] < v;
      toff[v] = o;
    }
    __syncthreads();
    for (int k = tid + 1; k <= N; k += kStreamThreads) {
      const int pa = tpar[k];
      int rank = 0;
      for (int k2 = 1; k2 < k; ++k2) rank += tpar[k2] == pa;
      tlist[toff[pa] + rank] = k;
    }
    __syncthreads();
    // the rows' records (written by the group's waves after their
    // streaming): lane l of wave wv reads row v = wv + 4 l; a record still
    // missing after spin_limit polls is computed here
    uint32_t soff[NPER];
    chunk_offsets(P.C, lane, kX1 * (int)sizeof(uint64_t), soff);
    const int v = wv + kStreamWaves * lane;
    const bool mine = v <= N;
    const Rsrc rs = __builtin_amdgcn_make_buffer_rsrc((void*)tree_rec(P, t0), (short)0,
                                                      (N + 1) * P.C * kPart * (int)sizeof(float), kRsrcWord3);
    const uint32_t off = (uint32_t)(mine ? v : 0) * (uint32_t)(P.C * kPart * (int)sizeof(float));
    int rowbad = 0;
    u32x4 w;
    for (int k = 0;; ++k) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the loads below are read again on every turn
      w = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kSC1);
      const bool ready = !mine || (w[1] == P.epoch && (v == 0 || w[3] == P.epoch));
      const uint64_t missing = __ballot(!ready);
      if (!missing) break;
      if (k > 2 * P.spin_limit + 16) {
        rowbad = 2;
        break;
      }
      if (k == P.spin_limit) {
        uint64_t m = missing;
        while (m) {
          const int l = __builtin_ctzll(m);
          m &= m - 1;
          const int vl = wv + kStreamWaves * l;
          if ((uint32_t)__builtin_amdgcn_readlane((int)w[1], l) != P.epoch)
            tree_row_job<DT, VEC, NPER>(P, t0 + vl, lane, soff);
          if (vl > 0 && (uint32_t)__builtin_amdgcn_readlane((int)w[3], l) != P.epoch)
            tree_row_job<DT, VEC, NPER>(P, t0 + tpar[vl], lane, soff);
        }
        __builtin_amdgcn_s_waitcnt(0);   // the records are in L2 before the poll below
      } else {
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (mine && rowbad == 0) {
      rowbad = (int)(w[0] >> kStatusShift);
      tamax[v] = (int)(w[0] & kTokMask);
      if (v > 0) tprob[v] = __uint_as_float(w[2]);
    }
    rowbad = wave_max_i(rowbad);
    if (lane == 0 && rowbad) atomicMax(&tst, rowbad);
    __syncthreads();
    bad = tst;
  }
  if (wv == 0) {
    int n = 0, tok = -1;
    if (!bad) {
      // the walk
      int v = 0, nr = 0;
      for (;;) {
        const int c0 = toff[v], c1 = toff[v + 1];
        int nxt = -1;
        float rem = 0.0f;
        nr = 0;
        for (int i = c0; i < c1; ++i) {
          const int k = tlist[i];
          const int x = ttok[k];
          bool acc;
          float p = 0.0f;
          if (sampled) {
            p = tprob[k];
            for (int j = 0; j < nr; ++j) p = trem[j] == x ? 0.0f : p;   // a token already removed has p 0
            acc = ld_const(P.uniforms, t0 + k - 1) * (1.0f - rem) < p;
          } else {
            acc = x == tamax[v];
          }
          if (acc) {
            nxt = k;
            break;
          }
          rem += p;
          trem[nr] = x;   // every lane writes the same value: each reads its own write
          trp[nr] = p;
          ++nr;
        }
        if (nxt < 0) break;
        tpath[n] = nxt;
        ++n;
        v = nxt;
      }
      if (!sampled) {
        tok = tamax[v];
      } else {
        // the final sample at v: the row's chunk masses less the removed candidates'
        const int r = t0 + v;
        uint32_t soff[NPER];
        chunk_offsets(P.C, lane, kX1 * (int)sizeof(uint64_t), soff);
        RowSlots<NPER> q;
        if (!tree_poll<DT, VEC, NPER>(P, r, 1, s, lane, soff, q)) {
          bad = 2;
        } else {
          float M, S;
          merge_row(q, P.C, 0, s, lane, M, S);
          float at[NPER], mt[NPER], tot[NPER];
          for (int pass = 0;; ++pass) {
            float ml = 0.0f;
#pragma unroll
            for (int jj = 0; jj < NPER; ++jj) {
              const int c = lane + 64 * jj;
              const bool inr = c < P.C;
              mt[jj] = inr ? slot_f(q.w[jj][0]) : -__builtin_huge_valf();
              at[jj] = inr ? chunk_scale(mt[jj], M, S, s) : 0.0f;
              float t = inr ? at[jj] * slot_f(q.w[jj][1]) : 0.0f;
              for (int j = 0; j < nr; ++j) t -= (inr && trem[j] / F::CH == c) ? trp[j] : 0.0f;
              tot[jj] = fmaxf(t, 0.0f);
              ml += tot[jj];
            }
            const float mass = wave_sum(ml);
            if (mass > 0.0f || nr == 0 || pass > 0) {
              // owner chunk: the first whose cumulative mass exceeds thr (rounding guard: the last with mass)
              const float thr = ld_const(P.uniforms, t0 + N) * mass;
              int cs = -1, last = -1;
              float before = 0.0f, last_before = 0.0f, base = 0.0f;
#pragma unroll
              for (int jj = 0; jj < NPER; ++jj) {
                const bool inr = lane + 64 * jj < P.C;
                const float t = inr ? tot[jj] : 0.0f;
                const float Gs = base + wave_scan(t, lane);
                const float Gex = Gs - t;
                const uint64_t hit = __ballot(inr && t > 0.0f && Gs > thr);
                const uint64_t pos = __ballot(inr && t > 0.0f);
                if (cs < 0 && hit) {
                  const int l = __builtin_ctzll(hit);
                  cs = 64 * jj + l;
                  before = lane_f(Gex, l);
                }
                if (pos) {
                  const int l = 63 - __builtin_clzll(pos);
                  last = 64 * jj + l;
                  last_before = lane_f(Gex, l);
                }
                base = lane_f(Gs, 63);
              }
              if (cs < 0) {
                cs = last;
                before = last_before;
              }
              if (cs < 0) {
                bad = 2;
              } else {
                const int ls = cs & 63, js = cs >> 6;
                const float tau = (thr - before) / lane_f(pick(at, js), ls);
                const float ct = chunk_offset(lane_f(pick(mt, js), ls), s);
                u32x4 R[2][kU];
                const int nb = P.V * F::ESIZE;
                issue_row<DT, VEC>(chunk_rsrc(P.target, r, P.tstride_b, cs, nb, true), lane, R[0]);
                tok = tree_scan<DT>(P, cs, tau, ct, s, trem, nr, lane, R);
                if (tok < 0) bad = 2;
              }
              break;
            }
            --nr;   // every mass removed (rounding): the residual before the last removal
          }
        }
      }
    }
    // outputs: the path's tokens and nodes, the final token, -1 after
    for (int j0 = 0; j0 <= N; j0 += 64) {
      const int j = j0 + lane;
      if (j <= N) {
        const int node = min(max(tpath[min(j, kMaxGamma)], 0), kMaxGamma);   // read for j < n only
        P.out_tokens[t0 + j] = (bad || j > n) ? -1 : j < n ? ttok[node] : tok;
        if (P.out_nodes) P.out_nodes[t0 + j] = (bad || j >= n) ? -1 : node;
      }
    }
    if (P.p_cand)
      for (int k = 1 + lane; k <= N; k += 64) P.p_cand[n0 + k - 1] = bad ? __builtin_nanf("") : tprob[k];
    if (lane == 0) P.acc_len[b] = bad == 2 ? -2 : bad ? -1 : n;
  }
  __syncthreads();   // the LDS arrays are reused by the next sequence
}

// ================================================================== the kernel

// D: the launch has draft logits (two-phase pipeline); otherwise phase 1
// alone, with the next item's loads in flight.
template <int DT, bool VEC, int NPER, bool D, bool TREE = false>
// Three waves per SIMD with draft logits (two for the rare element loads,
// whose larger register set would otherwise spill); at least seven for the
// token-only and plain sampling launches with 16-byte loads and rows of at
// most 128 chunks.
__global__ __launch_bounds__(kStreamThreads, D ? (VEC ? 3 : 2) : (VEC && !TREE && NPER < 4 ? 7 : 1)) void verify_kernel(Params P) {
  using F = Fmt<DT>;
  __shared__ uint32_t shres[kMaxGamma + 1];
  // the exponentials each wave keeps for its current item's phase 2
  // (launches with draft logits): e_d, and with HX the lower half of e_t
  constexpr int kKeep4 = kHalfInLds<NPER> ? 3 * F::L / 8 : F::L / 4;   // float4 per lane
  __shared__ float4 ssed[D ? kStreamWaves * kKeep4 * 64 : 1];
  // the lane from mbcnt, not from threadIdx.x, which then need not live
  // through the streaming loop
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = (int)(blockIdx.x % kGroups);
  const int wgl = (int)(blockIdx.x / kGroups);
  // The kernel arguments that the first logits loads depend on, requested
  // together here: left to the branches below, their scalar loads go out one
  // after another, a chain of round trips to a cold cache before any wave
  // issues its first load.
  __asm__ volatile("" ::"s"(P.gbounds), "s"(P.layout), "s"(P.rowinfo), "s"(P.target), "s"(P.draft),
                   "s"(P.tstride_b), "s"(P.dstride_b), "s"(P.C), "s"(P.Gw), "s"(P.V), "s"(P.gamma),
                   "s"(P.token_only), "s"(P.epoch), "s"(P.dummy), "s"(P.grow[grp]), "s"(P.grow[grp + 1]),
                   "s"(P.gseq[grp]), "s"(P.gseq[grp + 1]));
  __asm__ volatile("" ::"s"(P.div_c[0]), "s"(P.div_c[1]), "s"(P.div_c[2]), "s"(P.div_g[0]), "s"(P.div_g[1]),
                   "s"(P.div_g[2]));
  // An invalid layout leaves every group empty, so nothing streams; the flag
  // is acted on after the streaming loop, which keeps its read off the path
  // to the first loads.
  const bool bad_layout = P.gbounds != nullptr && ld_const(P.layout, 0) != P.epoch * 2u;
  const Group Gr = group_of(P, grp);
  const int n_items = (Gr.r1 - Gr.r0) * P.C;
  const int j = wgl * kStreamWaves + wave;
  const int G = P.Gw;
  // the wave's own dummy slots: waves never contend for a dummy cache line
  uint64_t* wdummy = P.dummy + ((int64_t)blockIdx.x * kStreamWaves + wave) * 8;
  if (j < n_items) {
    if (D) {
      uint32_t soff[NPER];
      chunk_offsets(P.C, lane, kX1 * (int)sizeof(uint64_t), soff);
      u32x4 R[2][kU];
      float EA[2][F::L], EB[2][F::L];
      float amt = 0.0f, amd = 0.0f, ast = 0.0f, bmt = 0.0f, bmd = 0.0f, bst = 0.0f;
      RowSlots<NPER> q;
      float4* sed = ssed + wave * kKeep4 * 64;   // e_d: L / 4 float4 per lane
      float4* sxt = sed + (F::L / 4) * 64;       // with HX, e_t's lower half: L / 8 float4 per lane
      // prologue: item 0 loaded and through phase 1, item 1 in flight
      Item ia = make_item(P, Gr.r0, j, n_items);
      Item ib = make_item(P, Gr.r0, j + G, n_items);
      issue_item<DT, VEC>(P, ia, lane, R);
      __builtin_amdgcn_sched_barrier(0);
      item_mode(P, ia);
      item_mode(P, ib);
      p1_item<DT, VEC>(P, ia, lane, wdummy, R, EA, amt, amd, ast, -1, VEC ? &ib : nullptr);
      if (ia.mode() == 1 && ia.pair()) keep_item<DT, kHalfInLds<NPER>>(EA, lane, sxt, sed);
      __builtin_amdgcn_sched_barrier(0);
      // Two steps per turn, one exit at the top: when the first step's item is
      // the wave's last, the second step runs on nothing (no waits, dummy writes).
      bool behind = true;   // (no row yet)
      for (int idx = j; idx < n_items; idx += 2 * G) {
        // cur = ia (EA), n1 = ib (in R), n2 = ic
        Item ic = make_item(P, Gr.r0, idx + 2 * G, n_items);
        step<DT, VEC, NPER>(P, lane, wdummy, soff, q, ia, EA[0], sxt, sed, amt, amd, ast, ib, R, EB, bmt, bmd, bst, ic,
                            behind);
        item_mode(P, ic);
        // cur = ib (EB), n1 = ic (in R), n2 = id
        Item id = make_item(P, Gr.r0, idx + 3 * G, n_items);
        step<DT, VEC, NPER>(P, lane, wdummy, soff, q, ib, EB[0], sxt, sed, bmt, bmd, bst, ic, R, EA, amt, amd, ast, id,
                            behind);
        item_mode(P, id);
        ia = ic;
        ib = id;
      }
    } else {
      u32x4 RA[2][kU], RB[2][kU];   // row 1 is never loaded or read
      float E[2][F::L];
      float mt, md, st;
      Item ia = make_item(P, Gr.r0, j, n_items);
      issue_target<DT, VEC>(P, ia, lane, RA[0]);
      item_mode(P, ia);
      for (int idx = j; idx < n_items; idx += 2 * G) {
        Item ib = make_item(P, Gr.r0, idx + G, n_items);
        issue_target<DT, VEC>(P, ib, lane, RB[0]);
        item_mode(P, ib);
        __builtin_amdgcn_sched_barrier(0);
        int x = -1;   // a token-only draft of this row: the chunk that holds it publishes e_t at x
        if (P.token_only && ia.mode() == 1 && ia.drafted()) x = ld_const(P.tokens, ia.rd());
        p1_item<DT, VEC, false>(P, ia, lane, wdummy, RA, E, mt, md, st, x);
        __builtin_amdgcn_sched_barrier(0);
        ia = make_item(P, Gr.r0, idx + 2 * G, n_items);
        issue_target<DT, VEC>(P, ia, lane, RA[0]);
        item_mode(P, ia);
        __builtin_amdgcn_sched_barrier(0);
        x = -1;
        if (P.token_only && ib.mode() == 1 && ib.drafted()) x = ld_const(P.tokens, ib.rd());
        p1_item<DT, VEC, false>(P, ib, lane, wdummy, RB, E, mt, md, st, x);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // loads of items past the end read zero-sized buffers; let them land
    __builtin_amdgcn_s_waitcnt(0);
  }
  if (bad_layout) {
    invalid_batch(P, wave * 64 + lane);   // from the wave and lane: threadIdx.x is not kept through the loop
    return;
  }
  if constexpr (TREE) {
    // the row jobs of the group's trees, spread over all its waves
    uint32_t soff[NPER];
    chunk_offsets(P.C, lane, kX1 * (int)sizeof(uint64_t), soff);
    for (int p = j; p < Gr.r1 - Gr.r0; p += P.Gw) tree_row_job<DT, VEC, NPER>(P, Gr.r0 + p, lane, soff);
  }
  // Resolution: sequence k of the group goes to workgroup Wg - 1 - (k mod Wg).
  // The last workgroups of a group stream one item fewer per wave when the
  // items do not divide evenly, so they finish streaming first.
  const int nseq = Gr.s1 - Gr.s0;
  for (int k = P.Wg - 1 - wgl; k < nseq; k += P.Wg) {
    if constexpr (TREE) resolve_tree<DT, VEC, NPER>(P, Gr.s0 + k, lane, wave);
    else resolve_sequence<DT, VEC, D, NPER>(P, Gr.s0 + k, lane, wave, shres);
  }
}

// ================================================================== commit kernel

// The commit of a verification step (see specverify_commit in the header):
// one wave per sequence appends its n + 1 emitted tokens to its token row.
struct CommitParams {
  int32_t B, gamma, R_d, capacity;
  const int32_t* cu_draft;   // NULL: uniform gamma
  const int32_t* acc_len;
  const int32_t* out_tokens;
  int32_t* seq_tokens;
  int64_t seq_stride;
  int32_t* seq_lens;
  int32_t* appended;         // may be NULL
  int32_t* next_token;       // may be NULL
};
constexpr int kCommitWaves = 4;

__global__ __launch_bounds__(64 * kCommitWaves) void commit_kernel(CommitParams C) {
  const int lane = threadIdx.x & 63;
  const int b = (int)blockIdx.x * kCommitWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (b >= C.B) return;
  int d0, gam;
  if (C.cu_draft == nullptr) {
    d0 = b * C.gamma;
    gam = C.gamma;
  } else {
    d0 = ld_const(C.cu_draft, b);
    gam = ld_const(C.cu_draft, b + 1) - d0;
  }
  const int n = ld_const(C.acc_len, b);
  // a length the layout does not allow, or a layout outside the run's rows,
  // counts as an invalid sequence: nothing outside the buffers is read
  const bool valid = n >= 0 && n <= gam && d0 >= 0 && d0 + gam <= C.R_d;
  const int k = n + 1;
  const int start = ld_const(C.seq_lens, b);
  const bool fits = valid && start >= 0 && start <= C.capacity - k;
  const int t0 = d0 + b;   // first target row of the sequence
  if (fits) {
    int32_t* row = C.seq_tokens + (int64_t)b * C.seq_stride + start;
    for (int j = lane; j < k; j += 64) row[j] = C.out_tokens[t0 + j];
  }
  if (lane == 0) {
    if (fits) C.seq_lens[b] = start + k;
    if (C.appended) C.appended[b] = fits ? k : valid ? -1 : 0;
    if (C.next_token) C.next_token[b] = fits ? C.out_tokens[t0 + n] : -1;
  }
}

// ================================================================== read probe (measurement)

// A plain streaming read of two byte ranges, and nothing else: the practical
// read bandwidth of the device for the bytes a run streams.  The ranges are
// cut into 4 KB chunks, read the way the verification kernel reads an item
// (one wave per chunk, four 16-byte nontemporal loads per lane through a
// buffer over the chunk, two chunks in flight per wave).  The words are
// XOR-folded per wave; the fold is stored to *sink only when it equals
// kProbeKey, a condition the compiler cannot decide, so no load is dropped.
constexpr int kProbeThreads = 256;
constexpr uint32_t kProbeKey = 0x9E3779B9u;
__device__ __forceinline__ Rsrc probe_chunk(const char* a, int64_t na, const char* b, int64_t nb, int64_t ca,
                                            int64_t k) {
  const bool in_a = k < ca;
  const int64_t off = (in_a ? k : k - ca) * kRowBytes;
  const int64_t n = in_a ? na - off : nb - off;   // <= 0 past the end: a zero-sized buffer
  return __builtin_amdgcn_make_buffer_rsrc((void*)((in_a ? a : b) + (n > 0 ? off : 0)), (short)0,
                                           n <= 0 ? 0 : (n > kRowBytes ? kRowBytes : (int)n), kRsrcWord3);
}
__global__ __launch_bounds__(kProbeThreads) void probe_kernel(const char* a, int64_t na, const char* b, int64_t nb,
                                                              uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kProbeThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kProbeThreads / 64);
  const int64_t ca = (na + kRowBytes - 1) / kRowBytes, nch = ca + (nb + kRowBytes - 1) / kRowBytes;
  uint32_t acc = 0;
  for (int64_t k0 = wave; k0 < nch; k0 += 2 * nwaves) {
    const Rsrc r0 = probe_chunk(a, na, b, nb, ca, k0);
    const Rsrc r1 = probe_chunk(a, na, b, nb, ca, k0 + nwaves);
    u32x4 w0[kU], w1[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) w0[u] = __builtin_amdgcn_raw_buffer_load_b128(r0, lane * 16 + u * 1024, 0, kNT);
#pragma unroll
    for (int u = 0; u < kU; ++u) w1[u] = __builtin_amdgcn_raw_buffer_load_b128(r1, lane * 16 + u * 1024, 0, kNT);
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= w0[u][0] ^ w0[u][1] ^ w0[u][2] ^ w0[u][3] ^ w1[u][0] ^ w1[u][1] ^ w1[u][2] ^ w1[u][3];
  }
  acc = (uint32_t)wave_max_i((int)acc) ^ (uint32_t)wave_min_i((int)acc);
  // a store that depends on every word keeps every load; it is taken only
  // for one fold value in 2^32 (one store per wave would serialise on the
  // one address)
  if (lane == 0 && acc == kProbeKey) sink[0] = acc;
}

// ================================================================== launch table

typedef void (*KernelFn)(Params);
// The three launches of a build: with draft logits, without (token-only
// drafts, or none), and draft trees (token-only candidates).
enum { kNoDraft = 0, kDraft = 1, kTree = 2 };
struct Kernels {
  KernelFn fn[3];
};
template <int DT, bool VEC, int NPER>
Kernels kernels_of() {
  return {{verify_kernel<DT, VEC, NPER, false>, verify_kernel<DT, VEC, NPER, true>,
           verify_kernel<DT, VEC, NPER, false, true>}};
}
template <int DT, bool VEC>
Kernels kernels_for(int nper) {
  if (nper == 1) return kernels_of<DT, VEC, 1>();
  if (nper == 2) return kernels_of<DT, VEC, 2>();
  // more than 128 chunks per row: fp32 only (the bf16 build would not fit
  // its registers)
  if constexpr (DT == SPECVERIFY_F32) return kernels_of<DT, VEC, 4>();
  return {{nullptr, nullptr, nullptr}};
}
Kernels kernels_for(int dtype, bool vec, int nper) {
  if (dtype == SPECVERIFY_F32) return vec ? kernels_for<SPECVERIFY_F32, true>(nper) : kernels_for<SPECVERIFY_F32, false>(nper);
  return vec ? kernels_for<SPECVERIFY_BF16, true>(nper) : kernels_for<SPECVERIFY_BF16, false>(nper);
}
int chunk_len(int dtype) { return dtype == SPECVERIFY_F32 ? Fmt<SPECVERIFY_F32>::CH : Fmt<SPECVERIFY_BF16>::CH; }
int chunks_for(int V, int dtype) { return (V + chunk_len(dtype) - 1) / chunk_len(dtype); }
int max_chunks(int dtype) { return dtype == SPECVERIFY_F32 ? kMaxChunks : kMaxChunksBf16; }
int nper_for(int C) { return C <= 64 ? 1 : C <= 128 ? 2 : 4; }
// Constants of udiv for the divisor d >= 1.
void udiv_consts(uint32_t d, uint32_t (&k)[3]) {
  int l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  k[0] = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
  k[1] = l < 1 ? l : 1;
  k[2] = l > 1 ? l - 1 : 0;
}

// ================================================================== host: checks and launch

// The limits of a configuration (see specverify_config); C = chunks per row.
specverify_status check_config(const specverify_config* cfg, int& C) {
  if (!cfg) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (cfg->max_batch < 1 || cfg->max_gamma < 0 || cfg->max_gamma > kMaxGamma || cfg->vocab < 1 ||
      cfg->spin_limit < 0 || (cfg->dtype != SPECVERIFY_F32 && cfg->dtype != SPECVERIFY_BF16))
    return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int64_t rows = (int64_t)cfg->max_batch * ((int64_t)cfg->max_gamma + 1);
  if (rows > (int64_t)1 << 24) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  C = chunks_for(cfg->vocab, cfg->dtype);
  if (C > max_chunks(cfg->dtype)) return SPECVERIFY_ERR_UNSUPPORTED;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device < 0 || cfg->device >= ndev)
    return SPECVERIFY_ERR_DEVICE;
  return SPECVERIFY_OK;
}
int spin_of(const specverify_config& cfg) {
  return cfg.spin_limit == 0 ? kDefaultSpin : cfg.spin_limit > kMaxSpin ? kMaxSpin : cfg.spin_limit;
}

// Residency of the persistent grids of a (dtype, nper) build on the current
// device: workgroups per CU times CUs, [vector loads][kind of launch].  With
// draft logits a row group needs at least C waves, so that the chunks of a
// row fall into one round or two consecutive ones and their waves meet in
// time.  A kernel that spilled to scratch would make the runtime allocate
// scratch at its first launch and spill in its inner loop: such a build is
// refused rather than run (hipErrorInvalidConfiguration).
hipError_t kernel_caps(int dtype, int nper, int C, int device, int (&cap)[2][3], int& capmax) {
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  capmax = 0;
  for (int v = 0; v < 6 && e == hipSuccess; ++v) {
    const int vec = v & 1, kind = v >> 1;
    const void* fn = (const void*)kernels_for(dtype, vec == 1, nper).fn[kind];
    hipFuncAttributes fa;
    e = hipFuncGetAttributes(&fa, fn);
    if (e == hipSuccess && fa.localSizeBytes > 0) e = hipErrorInvalidConfiguration;
    int per_cu = 0;
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kStreamThreads, 0);
    cap[vec][kind] = cus * per_cu;
    if (cap[vec][kind] > capmax) capmax = cap[vec][kind];
    if (e == hipSuccess && (per_cu < 1 || (kind == kDraft && (cap[vec][kind] / kGroups) * kStreamWaves < C)))
      e = hipErrorInvalidConfiguration;
  }
  return e;
}

// One run's launch: everything of Params but the workspace and the epoch.
struct Plan {
  Params P;
  KernelFn fn;
  bool ragged, has_dl;
  int64_t wg;     // workgroups per row group
  int64_t R_t;    // 0: an empty batch, nothing to launch
};

// The workspace of one launch (device memory).
struct Workspace {
  uint64_t* xch1;
  uint64_t* dummy;
  float* part;
  int4* rowinfo;
  uint32_t* layout;
  int32_t* gbounds;
};

// Check one run's arguments against a configuration (C chunks per row, at
// most max_rows target rows, resident workgroups cap) and plan its launch.
specverify_status plan_run(const specverify_config& cfg, int C, int nper, int64_t max_rows, const int (&cap)[2][3],
                           const specverify_inputs* in, const specverify_outputs* out, Plan& pl,
                           bool tree = false) {
  pl.R_t = 0;
  if (!in || !out) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int B = in->batch;
  if (B < 0 || B > cfg.max_batch) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (B == 0) return SPECVERIFY_OK;
  int64_t R_d;
  if (in->cu_draft == nullptr) {
    if (in->gamma < 0 || in->gamma > cfg.max_gamma) return SPECVERIFY_ERR_INVALID_ARGUMENT;
    R_d = (int64_t)B * in->gamma;
  } else {
    if (in->num_draft_rows < 0) return SPECVERIFY_ERR_INVALID_ARGUMENT;
    R_d = in->num_draft_rows;
  }
  const int64_t R_t = R_d + B;
  if (R_t > max_rows) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int V = cfg.vocab;
  if (!in->target_logits || !in->uniforms || !in->temperatures || !out->accepted_len ||
      !out->out_tokens)
    return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (R_d > 0 && !in->draft_tokens) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  // drafts without logits are token-only drafts: q_i = delta_{x_i}
  const bool has_dl = R_d > 0 && in->draft_logits != nullptr;
  if (in->target_stride < V || (has_dl && in->draft_stride < V)) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int esize = cfg.dtype == SPECVERIFY_F32 ? 4 : 2;
  if (in->target_stride * esize >= ((int64_t)1 << 31) || (has_dl && in->draft_stride * esize >= ((int64_t)1 << 31)))
    return SPECVERIFY_ERR_UNSUPPORTED;   // row strides of 2 GB or more
  if (((uintptr_t)in->target_logits % esize) || (has_dl && ((uintptr_t)in->draft_logits % esize)))
    return SPECVERIFY_ERR_UNSUPPORTED;   // logits must be element aligned
  // 16-byte loads need rows and the row length on 16-byte boundaries;
  // otherwise the kernels read element by element.
  const bool vec = !((uintptr_t)in->target_logits & 15) && !((in->target_stride * esize) & 15) &&
                   !(((int64_t)V * esize) & 15) &&
                   (!has_dl || (!((uintptr_t)in->draft_logits & 15) && !((in->draft_stride * esize) & 15)));

  const bool ragged = in->cu_draft != nullptr;
  Params& P = pl.P;
  P.target = (const char*)in->target_logits;
  P.draft = has_dl ? (const char*)in->draft_logits : nullptr;
  P.tstride_b = (uint32_t)(in->target_stride * esize);
  P.dstride_b = has_dl ? (uint32_t)(in->draft_stride * esize) : 0u;
  P.tokens = in->draft_tokens;
  P.uniforms = in->uniforms;
  P.temps = in->temperatures;
  P.cu_draft = in->cu_draft;
  // Row groups: contiguous ranges of whole sequences, about R_t / kGroups
  // target rows each (for a ragged batch the layout kernel splits it).
  int64_t rows_g;   // most target rows a group can get
  if (!ragged) {
    for (int g = 0; g <= kGroups; ++g) {
      P.gseq[g] = (int32_t)(((int64_t)g * B) / kGroups);
      P.grow[g] = P.gseq[g] * (in->gamma + 1);
    }
    rows_g = ((int64_t)(B + kGroups - 1) / kGroups) * (in->gamma + 1);
  } else {
    for (int g = 0; g <= kGroups; ++g) P.gseq[g] = P.grow[g] = 0;
    rows_g = (R_t + kGroups - 1) / kGroups + cfg.max_gamma + 1;
    if (rows_g > R_t) rows_g = R_t;
  }
  // Persistent grid: per row group, as many workgroups as the device holds,
  // never more than the busiest group has items for.
  const int64_t need = (rows_g * C + kStreamWaves - 1) / kStreamWaves;
  const int kind = tree ? kTree : has_dl ? kDraft : kNoDraft;
  int64_t wg = cap[vec ? 1 : 0][kind] / kGroups;
  if (wg > need) wg = need;
  if (wg < 1) wg = 1;
  P.gamma = ragged ? 0 : in->gamma;
  P.B = B;
  P.R_d = (int32_t)R_d;
  P.R_t = (int32_t)R_t;
  P.V = V;
  P.C = C;
  P.Gw = (int32_t)(wg * kStreamWaves);
  P.Wg = (int32_t)wg;
  P.max_gamma = cfg.max_gamma;
  P.spin_limit = spin_of(cfg);
  P.token_only = R_d > 0 && !has_dl && !tree;
  P.tree = tree;
  P.parents = nullptr;
  P.out_nodes = nullptr;
  P.p_cand = nullptr;
  udiv_consts((uint32_t)C, P.div_c);
  udiv_consts((uint32_t)(ragged ? 1 : in->gamma + 1), P.div_g);
  P.acc_len = out->accepted_len;
  P.out_tokens = out->out_tokens;
  P.p_draft = out->p_draft;
  P.q_draft = out->q_draft;
  P.beta = out->beta;
  P.resid = out->resid_mass;
  pl.fn = kernels_for(cfg.dtype, vec, nper).fn[kind];
  pl.ragged = ragged;
  pl.has_dl = has_dl;
  pl.wg = wg;
  pl.R_t = R_t;
  return SPECVERIFY_OK;
}

// The next epoch of a run on one workspace: never 0 (cleared memory carries
// tag 0) and below 2^31 (the layout flag holds epoch * 2).
uint32_t next_epoch(uint32_t& epoch) {
  if (++epoch == 0 || epoch >= 0x80000000u) epoch = 1;
  return epoch;
}

// Launch a planned run on stream (the current device is the workspace's).
hipError_t launch_plan(Plan& pl, const Workspace& w, uint32_t epoch, hipStream_t stream) {
  Params& P = pl.P;
  P.xch1 = w.xch1;
  P.dummy = w.dummy;
  P.part = w.part;
  P.rowinfo = pl.ragged ? w.rowinfo : nullptr;
  P.layout = w.layout;
  P.gbounds = pl.ragged ? w.gbounds : nullptr;
  P.epoch = epoch;
  if (pl.ragged)
    hipLaunchKernelGGL(layout_kernel, dim3(1), dim3(kLayoutThreads), 0, stream, P, w.rowinfo, w.gbounds, w.layout);
  hipLaunchKernelGGL(pl.fn, dim3((uint32_t)(pl.wg * kGroups)), dim3(kStreamThreads), 0, stream, P);
  return hipGetLastError();
}

// ================================================================== allocation-free runs

// Zeroes n 16-byte words with vector stores.
constexpr int kClearThreads = 256;
__global__ __launch_bounds__(kClearThreads) void clear_kernel(uint4* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kClearThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kClearThreads)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Host state of specverify_run_static, per device.
struct StaticDevice {
  char* base;              // the device's copy of scratch (its device address); null until set up
  uint32_t epoch;          // the last epoch used on the device
  bool cap_known[2][3];    // [dtype][nper 1, 2, 4]
  int cap[2][3][2][3];     // residency caps, as kernel_caps
};
constexpr int kStaticDevices = 64;
std::mutex g_static_mu;
StaticDevice g_static[kStaticDevices];

}  // namespace

// The workspace of specverify_run_static: a file-scope array that every
// device the library is loaded on holds until the process ends.  In host
// code its name stands for a host-side shadow, not for device memory: the
// host uses only the address hipGetSymbolAddress returns for each device.
static __device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

namespace {

// Set up specverify_run_static on the current device (once per device):
// the device's scratch address, and the scratch cleared on stream (tag 0 is
// never an epoch).
specverify_status static_setup(StaticDevice& d, hipStream_t stream) {
  if (d.base) return SPECVERIFY_OK;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SPECVERIFY_ERR_DEVICE;
  hipLaunchKernelGGL(clear_kernel, dim3(1024), dim3(kClearThreads), 0, stream, (uint4*)p,
                     (int64_t)(kScratchBytes / sizeof(uint4)));
  if (hipGetLastError() != hipSuccess) return SPECVERIFY_ERR_DEVICE;
  d.base = (char*)p;
  return SPECVERIFY_OK;
}

// specverify_run_static with its device current and the state lock held.
specverify_status run_static_locked(const specverify_config& cfg, int C, const specverify_inputs* in,
                                    const specverify_outputs* out, hipStream_t stream) {
  StaticDevice& d = g_static[cfg.device];
  specverify_status st = static_setup(d, stream);
  if (st != SPECVERIFY_OK) return st;
  const int nper = nper_for(C);
  const int ni = nper == 1 ? 0 : nper == 2 ? 1 : 2;
  if (!d.cap_known[cfg.dtype][ni]) {
    int capmax = 0;
    const hipError_t e = kernel_caps(cfg.dtype, nper, C, cfg.device, d.cap[cfg.dtype][ni], capmax);
    if (e != hipSuccess) return e == hipErrorInvalidConfiguration ? SPECVERIFY_ERR_UNSUPPORTED : SPECVERIFY_ERR_DEVICE;
    d.cap_known[cfg.dtype][ni] = true;
  }
  Plan pl;
  const int64_t max_rows = (int64_t)cfg.max_batch * ((int64_t)cfg.max_gamma + 1);
  st = plan_run(cfg, C, nper, max_rows, d.cap[cfg.dtype][ni], in, out, pl);
  if (st != SPECVERIFY_OK || pl.R_t == 0) return st;
  // this run's regions of the scratch, each on a 256-byte boundary
  size_t end = 0;
  auto take = [&end](size_t n) {
    const size_t at = end;
    end = (end + n + 255) & ~(size_t)255;
    return at;
  };
  const size_t rc = (size_t)pl.R_t * (size_t)C;
  const size_t o_x1 = take(rc * kX1 * sizeof(uint64_t));
  const size_t o_part = take(rc * kPart * sizeof(float));
  const size_t o_info = take((size_t)pl.R_t * sizeof(int4));
  const size_t o_dummy = take((size_t)pl.wg * kGroups * kStreamWaves * 8 * sizeof(uint64_t));
  const size_t o_layout = take(256);   // layout flag, group bounds at +64
  if (end > kScratchBytes) return SPECVERIFY_ERR_TOO_LARGE;
  const Workspace w{(uint64_t*)(d.base + o_x1),    (uint64_t*)(d.base + o_dummy), (float*)(d.base + o_part),
                    (int4*)(d.base + o_info),       (uint32_t*)(d.base + o_layout),
                    (int32_t*)(d.base + o_layout + 64)};
  return launch_plan(pl, w, next_epoch(d.epoch), stream) == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_ERR_DEVICE;
}

}  // namespace

struct specverify_ctx {
  specverify_config cfg;
  int chunks;
  int nper;
  int64_t rows;            // max target rows
  int cap[2][3];           // workgroups resident at once: [vector loads][kind of launch]
  void* ws;
  size_t ws_bytes;
  uint64_t* xch1;
  uint64_t* dummy;
  float* part;
  int4* rowinfo;
  uint32_t* layout;
  int32_t* gbounds;
  uint32_t epoch;
  int timing;              // recording events
  int trec;                // runs recorded since the measurement started
  hipEvent_t* ev;          // [SPECVERIFY_TIMING_RUNS][3], created on first use
};

extern "C" {

specverify_status specverify_create(const specverify_config* cfg, specverify_handle* out) {
  if (out) *out = nullptr;
  if (!cfg || !out) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  int C = 0;
  const specverify_status cst = check_config(cfg, C);
  if (cst != SPECVERIFY_OK) return cst;
  const int64_t rows = (int64_t)cfg->max_batch * ((int64_t)cfg->max_gamma + 1);
  specverify_ctx* h = new (std::nothrow) specverify_ctx();
  if (!h) return SPECVERIFY_ERR_OUT_OF_MEMORY;
  h->cfg = *cfg;
  h->cfg.spin_limit = spin_of(*cfg);
  h->chunks = C;
  h->nper = nper_for(C);
  h->rows = rows;
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (hipSetDevice(cfg->device) != hipSuccess) {
    delete h;
    return SPECVERIFY_ERR_DEVICE;
  }
  int capmax = 0;
  hipError_t e = kernel_caps(cfg->dtype, h->nper, C, cfg->device, h->cap, capmax);
  const size_t n1 = (size_t)rows * C * kX1 * sizeof(uint64_t);
  const size_t nd = (size_t)capmax * kStreamWaves * 8 * sizeof(uint64_t);   // dummy slots, per wave
  const size_t n2 = (size_t)rows * C * kPart * sizeof(float);
  const size_t n3 = (size_t)rows * sizeof(int4);
  const size_t n4 = 256;                                   // layout flag and group bounds
  h->ws_bytes = n1 + nd + n2 + n3 + n4;
  void* p = nullptr;
  if (e == hipSuccess) e = hipMalloc(&p, h->ws_bytes);
  if (e == hipSuccess) e = hipMemset(p, 0, h->ws_bytes);   // tag 0 is never an epoch
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipSetDevice(prev);
  if (e != hipSuccess) {
    if (p) (void)hipFree(p);
    delete h;
    return e == hipErrorOutOfMemory ? SPECVERIFY_ERR_OUT_OF_MEMORY
           : e == hipErrorInvalidConfiguration ? SPECVERIFY_ERR_UNSUPPORTED
                                               : SPECVERIFY_ERR_DEVICE;
  }
  h->ws = p;
  char* q = (char*)p;
  h->xch1 = (uint64_t*)q;
  h->dummy = (uint64_t*)(q + n1);
  h->part = (float*)(q + n1 + nd);
  h->rowinfo = (int4*)(q + n1 + nd + n2);
  h->layout = (uint32_t*)(q + n1 + nd + n2 + n3);
  h->gbounds = (int32_t*)(q + n1 + nd + n2 + n3 + 64);
  h->epoch = 0;
  h->timing = 0;
  h->trec = 0;
  h->ev = nullptr;
  *out = h;
  return SPECVERIFY_OK;
}

specverify_status specverify_run(specverify_handle h, const specverify_inputs* in,
                                 const specverify_outputs* out, void* hip_stream) {
  if (!h) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  Plan pl;
  const specverify_status st = plan_run(h->cfg, h->chunks, h->nper, h->rows, h->cap, in, out, pl);
  if (st != SPECVERIFY_OK || pl.R_t == 0) return st;
  const Workspace w{h->xch1, h->dummy, h->part, h->rowinfo, h->layout, h->gbounds};
  const uint32_t epoch = next_epoch(h->epoch);

  int prev = 0;
  (void)hipGetDevice(&prev);
  if (prev != h->cfg.device && hipSetDevice(h->cfg.device) != hipSuccess) return SPECVERIFY_ERR_DEVICE;
  hipStream_t stream = (hipStream_t)hip_stream;
  hipError_t e = hipSuccess;
  hipEvent_t* ev = nullptr;
  if (h->timing && h->trec < SPECVERIFY_TIMING_RUNS) ev = h->ev + 3 * h->trec++;
  if (ev) e = hipEventRecord(ev[0], stream);
  const hipError_t e2 = launch_plan(pl, w, epoch, stream);
  if (ev && e == hipSuccess) e = hipEventRecord(ev[1], stream);
  if (ev && e == hipSuccess) e = hipEventRecord(ev[2], stream);
  if (prev != h->cfg.device) (void)hipSetDevice(prev);
  return (e == hipSuccess && e2 == hipSuccess) ? SPECVERIFY_OK : SPECVERIFY_ERR_DEVICE;
}

specverify_status specverify_run_tree(specverify_handle h, const specverify_tree_inputs* in,
                                      const specverify_tree_outputs* out, void* hip_stream) {
  if (!h || !in || !out) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (in->batch > 0 && in->cu_nodes == nullptr) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (in->num_nodes > 0 && in->parents == nullptr) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  // a tree batch is a ragged batch of target rows without draft logits
  specverify_inputs li;
  li.batch = in->batch;
  li.gamma = 0;
  li.cu_draft = in->cu_nodes;
  li.num_draft_rows = in->num_nodes;
  li.target_logits = in->target_logits;
  li.target_stride = in->target_stride;
  li.draft_logits = nullptr;
  li.draft_stride = 0;
  li.draft_tokens = in->tokens;
  li.uniforms = in->uniforms;
  li.temperatures = in->temperatures;
  specverify_outputs lo;
  lo.accepted_len = out->accepted_len;
  lo.out_tokens = out->out_tokens;
  lo.p_draft = lo.q_draft = lo.beta = lo.resid_mass = nullptr;
  Plan pl;
  const specverify_status st = plan_run(h->cfg, h->chunks, h->nper, h->rows, h->cap, &li, &lo, pl, true);
  if (st != SPECVERIFY_OK || pl.R_t == 0) return st;
  pl.P.parents = in->parents;
  pl.P.out_nodes = out->out_nodes;
  pl.P.p_cand = out->p_cand;
  const Workspace w{h->xch1, h->dummy, h->part, h->rowinfo, h->layout, h->gbounds};
  const uint32_t epoch = next_epoch(h->epoch);
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (prev != h->cfg.device && hipSetDevice(h->cfg.device) != hipSuccess) return SPECVERIFY_ERR_DEVICE;
  const hipError_t e = launch_plan(pl, w, epoch, (hipStream_t)hip_stream);
  if (prev != h->cfg.device) (void)hipSetDevice(prev);
  return e == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_ERR_DEVICE;
}

specverify_status specverify_run_static(const specverify_config* cfg, const specverify_inputs* in,
                                        const specverify_outputs* out, void* hip_stream) {
  int C = 0;
  const specverify_status cst = check_config(cfg, C);
  if (cst != SPECVERIFY_OK) return cst;
  if (cfg->device >= kStaticDevices) return SPECVERIFY_ERR_UNSUPPORTED;
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (prev != cfg->device && hipSetDevice(cfg->device) != hipSuccess) return SPECVERIFY_ERR_DEVICE;
  specverify_status st;
  {
    std::lock_guard<std::mutex> lock(g_static_mu);
    st = run_static_locked(*cfg, C, in, out, (hipStream_t)hip_stream);
  }
  if (prev != cfg->device) (void)hipSetDevice(prev);
  return st;
}

specverify_status specverify_commit(specverify_handle h, const specverify_commit_args* a, void* hip_stream) {
  if (!h || !a) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int B = a->batch;
  if (B < 0 || B > h->cfg.max_batch) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (B == 0) return SPECVERIFY_OK;
  int64_t R_d;
  if (a->cu_draft == nullptr) {
    if (a->gamma < 0 || a->gamma > h->cfg.max_gamma) return SPECVERIFY_ERR_INVALID_ARGUMENT;
    R_d = (int64_t)B * a->gamma;
  } else {
    if (a->num_draft_rows < 0) return SPECVERIFY_ERR_INVALID_ARGUMENT;
    R_d = a->num_draft_rows;
  }
  if (R_d + B > h->rows) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (!a->accepted_len || !a->out_tokens || !a->seq_tokens || !a->seq_lens || a->capacity < 0 ||
      a->seq_stride < a->capacity)
    return SPECVERIFY_ERR_INVALID_ARGUMENT;
  CommitParams C;
  C.B = B;
  C.gamma = a->cu_draft ? 0 : a->gamma;
  C.R_d = (int32_t)R_d;
  C.capacity = a->capacity;
  C.cu_draft = a->cu_draft;
  C.acc_len = a->accepted_len;
  C.out_tokens = a->out_tokens;
  C.seq_tokens = a->seq_tokens;
  C.seq_stride = a->seq_stride;
  C.seq_lens = a->seq_lens;
  C.appended = a->appended;
  C.next_token = a->next_token;
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (prev != h->cfg.device && hipSetDevice(h->cfg.device) != hipSuccess) return SPECVERIFY_ERR_DEVICE;
  hipLaunchKernelGGL(commit_kernel, dim3((uint32_t)((B + kCommitWaves - 1) / kCommitWaves)),
                     dim3(64 * kCommitWaves), 0, (hipStream_t)hip_stream, C);
  const hipError_t e = hipGetLastError();
  if (prev != h->cfg.device) (void)hipSetDevice(prev);
  return e == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_ERR_DEVICE;
}

specverify_status specverify_destroy(specverify_handle h) {
  if (!h) return SPECVERIFY_OK;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(h->cfg.device);
  if (h->ev)
    for (int k = 0; k < 3 * SPECVERIFY_TIMING_RUNS; ++k) (void)hipEventDestroy(h->ev[k]);
  delete[] h->ev;
  (void)hipFree(h->ws);
  (void)hipSetDevice(prev);
  delete h;
  return SPECVERIFY_OK;
}

specverify_status specverify_set_timing(specverify_handle h, int32_t enable) {
  if (!h) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (enable && !h->ev) {
    int prev = 0;
    (void)hipGetDevice(&prev);
    if (hipSetDevice(h->cfg.device) != hipSuccess) return SPECVERIFY_ERR_DEVICE;
    hipEvent_t* ev = new (std::nothrow) hipEvent_t[3 * SPECVERIFY_TIMING_RUNS];
    int n = 0;
    hipError_t e = ev ? hipSuccess : hipErrorOutOfMemory;
    for (; e == hipSuccess && n < 3 * SPECVERIFY_TIMING_RUNS; ++n) e = hipEventCreate(&ev[n]);
    (void)hipSetDevice(prev);
    if (e != hipSuccess) {
      for (int k = 0; k < n - 1; ++k) (void)hipEventDestroy(ev[k]);
      delete[] ev;
      return SPECVERIFY_ERR_DEVICE;
    }
    h->ev = ev;
  }
  h->timing = enable ? 1 : 0;
  if (enable) h->trec = 0;
  return SPECVERIFY_OK;
}

specverify_status specverify_timing_totals(specverify_handle h, int32_t* runs, float* stream_ms,
                                           float* finish_ms) {
  if (!h || !runs || !stream_ms || !finish_ms) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  *runs = 0;
  *stream_ms = 0.0f;
  *finish_ms = 0.0f;
  if (h->trec == 0) return SPECVERIFY_OK;
  const hipEvent_t* ev = h->ev;
  if (hipEventSynchronize(ev[3 * (h->trec - 1) + 2]) != hipSuccess) return SPECVERIFY_ERR_DEVICE;
  double a = 0.0, f = 0.0;
  for (int k = 0; k < h->trec; ++k) {
    float x = 0.0f, y = 0.0f;
    if (hipEventElapsedTime(&x, ev[3 * k], ev[3 * k + 1]) != hipSuccess ||
        hipEventElapsedTime(&y, ev[3 * k + 1], ev[3 * k + 2]) != hipSuccess)
      return SPECVERIFY_ERR_DEVICE;
    a += x;
    f += y;
  }
  *runs = h->trec;
  *stream_ms = (float)a;
  *finish_ms = (float)f;
  h->trec = 0;
  return SPECVERIFY_OK;
}

specverify_status specverify_probe_read(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes,
                                        uint32_t* sink, void* hip_stream) {
  if (!sink || a_bytes < 0 || b_bytes < 0 || (a_bytes > 0 && !a) || (b_bytes > 0 && !b) || (a_bytes % 16) ||
      (b_bytes % 16) || ((uintptr_t)a % 16) || ((uintptr_t)b % 16))
    return SPECVERIFY_ERR_INVALID_ARGUMENT;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return SPECVERIFY_ERR_DEVICE;
  const int64_t chunks = (a_bytes + kRowBytes - 1) / kRowBytes + (b_bytes + kRowBytes - 1) / kRowBytes;
  int64_t grid = (int64_t)cus * 8;   // eight workgroups of four waves per CU
  const int64_t need = (chunks + 2 * (kProbeThreads / 64) - 1) / (2 * (kProbeThreads / 64));
  if (grid > need) grid = need;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(probe_kernel, dim3((uint32_t)grid), dim3(kProbeThreads), 0, (hipStream_t)hip_stream,
                     (const char*)a, a_bytes, (const char*)b, b_bytes, sink);
  return hipGetLastError() == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_ERR_DEVICE;
}

int32_t specverify_chunks_per_row(specverify_handle h) { return h ? h->chunks : 0; }
int64_t specverify_workspace_bytes(specverify_handle h) { return h ? (int64_t)h->ws_bytes : 0; }

}  // extern "C"
