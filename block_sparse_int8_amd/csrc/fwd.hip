// Block-sparse attention forward (gfx950): the INT8 path and the floating-QK
// path, one kernel templated on the score type.
//
// Configure Sol Sparse Attention, "How it works": kept key blocks are computed
// exactly on the INT8 Q/K (the W8A8 integer path) or, with a floating dense
// backend, on the bf16 Q/K; skipped blocks contribute their centroids to the
// same online softmax (Configure H3 Static Virtual KV, mode list, "residual").
// FlashVSR Sparge Attention, "How it works": one sparse call over the whole
// compact block map.
//
// Mapping onto CDNA4:
//  * One workgroup (4 waves, 256 threads) per 128-row query block, two per CU;
//    wave w owns query rows 32w..32w+31.  Its Q fragment stays in registers
//    for the whole kernel.
//  * Exact 64-key tiles: K and V are copied straight into LDS (buffer loads
//    into LDS, rows XOR-swizzled instead of padded); S^T = K.Q^T with
//    v_mfma_i32_32x32x32_i8 (INT8) or v_mfma_f32_32x32x16_bf16 (bf16), so
//    each lane ends up holding one query row's scores — the layout the PV
//    product needs as its B operand, with no LDS round trip.
//    O^T = V^T.P^T with v_mfma_f32_32x32x16_bf16; the V^T operand comes
//    straight from the row-major V tile through ds_read_b64_tr_b16.
//  * The tiles run as a software pipeline over 32-key halves: each step puts
//    the next half's QK^T and the previous half's PV on the matrix cores and
//    computes the current half's weights in their shadow (pipe_step).
//  * Softmax in base 2 with sm_scale*log2(e) folded into the per-tile scale
//    (a_i*b_j on the INT8 path); the running max is shared by the two lanes
//    (l, l^32) that hold the same query row and lags the scores while the
//    weights stay small; row sums stay per lane until the end.
//  * Centroid columns are batched 32 at a time into the same tile shapes, as
//    bf16 hi+lo pairs (about 16 mantissa bits), with log2(count) added to the
//    logit so a centroid weighs as much as the keys it stands for.
//  * The grid walks query blocks XCD by XCD (block id b lands on XCD b % 8), so
//    the query blocks of one head share that XCD's L2 while they stream the same
//    K/V tiles.
#include "sa_device.h"
#include "sa_launch.h"

#include <limits.h>

namespace sa {

namespace {

constexpr int kWin = 512;      // map entries scanned per list-building window
constexpr float kLazy = 8.0f;  // rescale O only when the row max grows by more than 2^8

// LDS layout of the K and V tiles and of the centroid staging: unpadded rows
// with their 16-byte units (K) or 64-byte segments (V) permuted per row by an
// XOR, so the readers' access patterns hit distinct banks without padding:
//  * K rows are read with ds_read_b128, 16 lanes per cycle on 16 consecutive
//    rows at the same logical unit; a 256-byte bank line holds 256/KROW rows,
//    and rows of one line get their units XORed with different values.
//  * V rows are read with ds_read_b64_tr_b16, 16 lanes per cycle on 4
//    consecutive rows x 32 bytes; rows of different lines sharing the bank
//    positions get their 64-byte segments XORed with different values.
// Every row's data stays inside its own row, so a whole tile is one
// contiguous run of 1 KiB copy chunks (no padding lanes).
template <int D, int KB = 1>
struct FwdLds {
  static constexpr int KROW = KB * D;         // K tile row (bytes): int8 (KB = 1) or bf16 (KB = 2)
  static constexpr int VROW = 2 * D;          // bf16 V tile row (bytes)
  static constexpr int KCROW = 2 * D;         // bf16 centroid-K row (bytes)
  static constexpr int KU = KROW / 16;        // 16-byte units per K row = 1 KiB copies per K tile
  static constexpr int VU = VROW / 16;        // 16-byte units per V row = 1 KiB copies per V tile
  static constexpr int KST = kTile * KROW;    // one K stage
  static constexpr int VST = kTile * VROW;    // one V stage
  // centroid staging: K hi/lo in V stage 0, V hi/lo in V stage 1
  static constexpr int KCL_OFF = 32 * KCROW;
  static constexpr int VCL_OFF = 32 * VROW;
  static_assert(2 * 32 * KCROW <= VST && 2 * 32 * VROW <= VST, "centroid staging must fit a V stage");
  static_assert(KU % 4 == 0 && VU % 4 == 0, "tile copies split evenly over 4 waves");
  // byte offset of (row r, byte x of the row) in a K tile / V tile / centroid-K staging
  __device__ __forceinline__ static constexpr int k_off(int r, int x) {
    return r * KROW + (((x >> 4) ^ ((r / (256 / KROW)) & (KU - 1))) << 4) + (x & 15);
  }
  __device__ __forceinline__ static constexpr int v_off(int r, int x) {
    return r * VROW + (((x >> 6) ^ ((r / (VROW >= 256 ? 1 : 256 / VROW)) & (VROW / 64 - 1))) << 6) + (x & 63);
  }
  __device__ __forceinline__ static constexpr int kc_off(int r, int x) {
    return r * KCROW + (((x >> 4) ^ ((r / (KCROW >= 256 ? 1 : 256 / KCROW)) & (KCROW / 16 - 1))) << 4) + (x & 15);
  }
};

__device__ __forceinline__ v4bf tr16(const uint8_t* lds_byte_ptr) {
  v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS v4s*)(lds_byte_ptr));
  return __builtin_bit_cast(v4bf, r);
}

__device__ __forceinline__ v8bf cat8(v4bf a, v4bf b) {
  return (v8bf){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// A lane offset passed through an empty asm statement: LDS addresses are then
// formed as stage + offset + constant, a derivation short enough for the
// compiler to keep track of which LDS variable each read touches (it only
// follows a few pointer steps).  Without that knowledge it would make every
// such read wait for all direct LDS copies in flight.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// 8 int8 codes (two dwords) -> 8 bf16 (exact: |code| <= 127).
__device__ __forceinline__ v8bf i8x8_to_bf16(int lo, int hi) {
  v8bf r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)(float)(int8_t)((lo >> (8 * e)) & 0xFF);
    r[4 + e] = (__bf16)(float)(int8_t)((hi >> (8 * e)) & 0xFF);
  }
  return r;
}

// max of a value over the lane pair (l, l^32), which hold the same query row.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Lazy online-softmax rescale: the running max m_run only moves when a tile's
// max exceeds it by more than kLazy (so exp2(x - m_run) <= 2^kLazy, safe in
// bf16 and fp32); the wave takes the branch if any of its rows needs it.
template <int NS>
__device__ __forceinline__ void maybe_rescale(float m_tile, float& m_run, float& l_run, v16f (&O)[NS]) {
  const bool need = m_tile > m_run + kLazy;
  if (__ballot(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.0f;
    if (need) m_run = m_tile;
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < NS; ++c) O[c] *= alpha;
  }
}

// Direct copy into LDS of one 64-row K tile (int8) and, unless V arrives as
// INT8, one 64-row V tile (bf16) with buffer_load_dwordx4 ... lds.  Lane L of
// a wave instruction lands at LDS offset 16*L of that instruction's 1 KiB
// chunk, so the permuted row layout is produced by picking each lane's
// source.  The per-lane source offsets do not depend on the tile and are
// computed once; the tile offset is a scalar.
template <int D, int KB>
struct DmaPlan {
  static constexpr int KI = FwdLds<D, KB>::KU / 4;   // K copies per wave
  static constexpr int VI = FwdLds<D, KB>::VU / 4;   // V copies per wave
  uint32_t koff[KI];   // unsigned: the copy uses a scalar base plus a 32-bit lane offset
  uint32_t voff[VI];
};

// Lane L of copy chunk c lands at byte 1024c + 16L of the stage; its source is
// the 16 bytes the layout puts there (XOR is its own inverse, so the logical
// unit is the stored one XORed with the row's value).
template <int D, int KB>
__device__ __forceinline__ DmaPlan<D, KB> make_dma_plan(int wave, int lane) {
  using L = FwdLds<D, KB>;
  DmaPlan<D, KB> pl;
#pragma unroll
  for (int t = 0; t < DmaPlan<D, KB>::KI; ++t) {
    const int pos = (wave + 4 * t) * 1024 + 16 * lane, row = pos / L::KROW;
    pl.koff[t] = (uint32_t)(row * L::KROW + (L::k_off(row, pos % L::KROW) - row * L::KROW));
  }
#pragma unroll
  for (int t = 0; t < DmaPlan<D, KB>::VI; ++t) {
    const int pos = (wave + 4 * t) * 1024 + 16 * lane, row = pos / L::VROW;
    pl.voff[t] = (uint32_t)(row * L::VROW + (L::v_off(row, pos % L::VROW) - row * L::VROW));
  }
  return pl;
}

// INT8 V (FlashVSR's INT8 cache) goes through registers so it can be widened
// to bf16 exactly before it is written to LDS.
template <int D>
struct VRegs {
  v4i r[D / 64];
};

template <int D>
__device__ __forceinline__ void load_v_int8(const int8_t* vsrc, VRegs<D>& vr, int tid) {
#pragma unroll
  for (int e = 0; e < D / 64; ++e) {
    const int v = tid + 256 * e, r = v / (D / 16), cc = v % (D / 16);
    vr.r[e] = *reinterpret_cast<const v4i*>(vsrc + r * D + cc * 16);
  }
}

// The LDS addresses are formed from the thread index at each call (opaque to
// the compiler): kept live across the tile loop instead, they would be spilled.
template <int D>
__device__ __forceinline__ void store_v_int8(uint8_t* vbuf, const VRegs<D>& vr, int tid) {
  using L = FwdLds<D>;
  tid = opaque(tid);
#pragma unroll
  for (int e = 0; e < D / 64; ++e) {
    const int v = tid + 256 * e, r = v / (D / 16), cc = v % (D / 16);
    *reinterpret_cast<v8bf*>(vbuf + L::v_off(r, cc * 32)) = i8x8_to_bf16(vr.r[e][0], vr.r[e][1]);
    *reinterpret_cast<v8bf*>(vbuf + L::v_off(r, cc * 32 + 16)) = i8x8_to_bf16(vr.r[e][2], vr.r[e][3]);
  }
}

// One 16-byte direct load per lane into LDS (buffer_load_dwordx4 ... lds):
// the lane's 16 bytes, at byte voff + soff of the buffer, land at LDS byte
// address lds_addr + 16 * lane.  The buffer form takes a scalar base and a
// 32-bit lane offset that does not change from tile to tile, so a copy costs
// no vector instructions; loads past the buffer's end return zeros.  The LDS
// address is passed as a plain wave-uniform integer that the compiler cannot
// trace to an LDS variable: it then keeps the copy in order with every LDS
// access but adds no wait of its own for it before later LDS reads.  The tile
// loop's barriers wait for the copies (vmcnt(0) before each __syncthreads),
// and no LDS read touches a stage while its copy is in flight.  Kept out of
// templates: the host compilation pass only accepts the builtin in a plain
// function.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                          uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("" : "+s"(lds_addr));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (SA_LDS void*)(uintptr_t)lds_addr, 16, voff, soff, 0, 0);
}

// Buffer resource over num_bytes at base (raw, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(SA_LDS const void*)p;
}

// Scalars of one exact tile, loaded a tile or more before they are used, so
// the compute never waits on them: the loads are consumed after a later
// barrier (which waits for all of this wave's loads).
struct TileInfo {
  int krow0;
  int vblk;               // V block of the tile: raw table entry when V rows are remapped (clamped when used)
  int nvb;                // V blocks of the tensor (clamp bound), 0 when V rows are not remapped
  float kscale, pscale;
  __device__ __forceinline__ int vrow0() const {
    // the entry is wave-uniform: clamp it on the scalar unit
    const int v = __builtin_amdgcn_readfirstlane(vblk);
    const int vb = nvb > 0 ? min(max(v, 0), nvb - 1) : v;
    return vb * kTile;
  }
};

// The loads are only issued here: nothing waits for them until the tile is
// used, an iteration later (the V table entry is clamped then too).  Scale
// indices are shifts (k_scale_rows and v_scale_rows are 64 or 128).
template <bool QF, bool VI8>
__device__ __forceinline__ TileInfo fetch_tile(const FwdArgs& a, int64_t bh, int kt, int nKS, int nVS) {
  TileInfo t;
  t.krow0 = kt * kTile;
  t.nvb = a.v_block_src ? a.Lv / kTile : 0;
  t.vblk = a.v_block_src ? a.v_block_src[kt] : kt;
  t.kscale = QF ? 1.0f : a.k_scale[bh * nKS + (t.krow0 >> a.ks_shift)];
  // INT8 V needs its block's scale, which depends on the table entry
  t.pscale = VI8 ? a.v_scale[bh * nVS + ((t.vrow0()) >> a.vs_shift)] : 1.0f;
  return t;
}

// The copy of one tile into a stage, issued piecewise: K (and bf16 V) by
// direct loads, INT8 V into registers (written to LDS later by store_v_int8).
// A wave owns K instructions wave + 4u (u < KI) and V instructions wave + 4u
// (u < VI).  The tile loop hands this to the compute of the current tile,
// which issues the pieces between its matrix-core segments: issued in one
// burst, the copies of all waves on a CU queue behind each other in the
// vector-memory path and stall the waves' in-order issue.  Every piece is
// branch-free (wave is wave-uniform, every wave owns the same number of
// chunks), so the pieces do not split the compute into separately scheduled
// blocks.
template <int D, int KB, bool VI8>
struct TileCopy {
  static constexpr int KI = DmaPlan<D, KB>::KI;
  static constexpr int VI = VI8 ? 0 : DmaPlan<D, KB>::VI;
  static constexpr int PIECES = KI + VI;   // direct loads per wave for one K tile and one V tile
  __amdgpu_buffer_rsrc_t krs, vrs;   // K (int8) and bf16 V of this head
  uint32_t koff, voff;               // byte offsets of the K tile's / V tile's first row
  uint32_t klds, vlds;               // destination K and V stages (LDS byte addresses)
  const DmaPlan<D, KB>* plan;
  int wave;                          // wave-uniform, 0..3
  __device__ __forceinline__ void k(int u) const {
    lds_dma16(krs, plan->koff[u], koff, klds + (wave + 4 * u) * 1024);
  }
  __device__ __forceinline__ void v(int u) const {
    lds_dma16(vrs, plan->voff[u], voff, vlds + (wave + 4 * u) * 1024);
  }
  // piece p < KI: K load p; otherwise V load p - KI
  __device__ __forceinline__ void piece(int p) const {
    if (p < KI) k(p);
    else if (p < PIECES) v(p - KI);
  }
  __device__ __forceinline__ void all_k() const {
#pragma unroll
    for (int u = 0; u < KI; ++u) k(u);
  }
  __device__ __forceinline__ void all() const {
#pragma unroll
    for (int p = 0; p < PIECES; ++p) piece(p);
  }
};

// Copy of the K tile of tk and the V tile of tv (bf16 V only) into the given
// stages.
template <int D, int KB, bool VI8>
__device__ __forceinline__ TileCopy<D, KB, VI8> tile_copy(const TileInfo& tk, const TileInfo& tv, uint8_t* kbuf,
                                                          uint8_t* vbuf, __amdgpu_buffer_rsrc_t krs,
                                                          __amdgpu_buffer_rsrc_t vrs, const DmaPlan<D, KB>& plan,
                                                          int wave) {
  return TileCopy<D, KB, VI8>{krs,
                          vrs,
                          (uint32_t)(tk.krow0 * KB * D),
                          (uint32_t)(tv.vrow0() * D * 2),
                          lds_address(kbuf),
                          lds_address(vbuf),
                          &plan,
                          wave};
}

// Wait for this wave's direct copies, then for the whole workgroup: after it,
// every copy issued before it by any wave has landed in LDS.
__device__ __forceinline__ void copies_done_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Scores leave the integer MFMA already in float form: the accumulators start
// at the bit pattern of 1.5 * 2^23, whose float spacing is 1, so the finished
// int32 accumulator read as a float is exactly 1.5 * 2^23 + S while
// |S| < 2^21 (|S| <= 127 * 127 * d < 2^21 for d <= 128).
constexpr int kMagicI = 0x4B400000;
constexpr float kMagicF = 12582912.0f;
// Fast-path acceptance bound on a lane's partial row sum (each weight is at
// most this, so every weight stays far from fp32/bf16 overflow).
constexpr float kFastSum = 4096.0f;

// Score accumulators: int32 for the INT8 products (seeded with kMagicI, read
// as float), fp32 for the floating ones.
template <bool QF>
struct ScoreAcc {
  using type = v16i;
};
template <>
struct ScoreAcc<true> {
  using type = v16f;
};
template <bool QF>
using SAcc = typename ScoreAcc<QF>::type;

// Score e of a half as the float the weight FMA takes: 1.5*2^23 + S for the
// INT8 products, the fp32 dot for the floating ones.
__device__ __forceinline__ float score_f(const v16i& acc, int e) { return __int_as_float(acc[e]); }
__device__ __forceinline__ float score_f(const v16f& acc, int e) { return acc[e]; }

// The addend of the weight FMA, exp2(x*c + b) = exp2(S*c - m): it absorbs the
// 1.5*2^23 offset of the INT8 scores.
template <bool QF>
__device__ __forceinline__ float weight_bias(float c, float m) {
  return QF ? -m : -__builtin_fmaf(kMagicF, c, m);
}

// p = exp2(S*c - m) for the 16 scores a lane holds in one 32-key half of the
// tile, as bf16 pairs (INT8 V: scaled by the V block scale before rounding);
// b = weight_bias(c, m) is formed once per row, so each weight is one FMA and
// one exp2.  Returns the lane's row-sum part: the bf16-rounded weights (bf16
// V) or the unrounded unscaled ones (INT8 V).
template <bool VI8, bool MASKED, class Acc>
__device__ __forceinline__ float half_weights(const Acc& acc, int key0, float c, float b, float pscale, int nvalid,
                                              int hh, uint32_t (&pw)[8]) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(score_f(acc, 2 * e), c, b));
    float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(score_f(acc, 2 * e + 1), c, b));
    if (MASKED) {
      const int k0 = key0 + ((2 * e) / 4) * 8 + hh * 4 + (2 * e) % 4;
      p0 = k0 < nvalid ? p0 : 0.0f;
      p1 = k0 + 1 < nvalid ? p1 : 0.0f;
    }
    v2bf pk;
    if (VI8) {
      psum += p0 + p1;
      pk = (v2bf){(__bf16)(p0 * pscale), (__bf16)(p1 * pscale)};
    } else {
      pk = (v2bf){(__bf16)p0, (__bf16)p1};
      psum = __builtin_amdgcn_fdot2_f32_bf16(pk, (v2bf){(__bf16)1.0f, (__bf16)1.0f}, psum, false);
    }
    pw[e] = __builtin_bit_cast(uint32_t, pk);
  }
  return psum;
}

// Row max over a half's scores in score*c units (the lane pair l, l^32 holds
// one query row); -inf when none of them is valid.
template <bool MASKED>
__device__ __forceinline__ float half_max(const v16i& acc, int key0, float c, int nvalid, int hh) {
  int mi = INT_MIN;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    int v = acc[e];
    if (MASKED) v = key0 + (e / 4) * 8 + hh * 4 + (e % 4) < nvalid ? v : INT_MIN;
    mi = max(mi, v);
  }
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)mi, (unsigned)mi, false, false);
  mi = max((int)r[0], (int)r[1]);
  return mi == INT_MIN ? -INFINITY : (float)(mi - kMagicI) * c;
}
template <bool MASKED>
__device__ __forceinline__ float half_max(const v16f& acc, int key0, float c, int nvalid, int hh) {
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float v = acc[e];
    if (MASKED) v = key0 + (e / 4) * 8 + hh * 4 + (e % 4) < nvalid ? v : -INFINITY;
    mx = fmaxf(mx, v);
  }
  mx = pair_max(mx);
  return mx == -INFINITY ? -INFINITY : mx * c;
}

// Exact online-softmax step for one 32-key half: the half's row max moves
// m_run lazily, then the weights are computed against it.  Returns the lane's
// row-sum part.
template <int NS, bool VI8, bool MASKED, bool QF>
__device__ __forceinline__ float half_exact(const SAcc<QF>& acc, int key0, float c, float pscale, int nvalid, int hh,
                                            v16f (&O)[NS], float& m_run, float& l_run, uint32_t (&pw)[8]) {
  maybe_rescale<NS>(half_max<MASKED>(acc, key0, c, nvalid, hh), m_run, l_run, O);
  // rows with no valid key so far keep m_run = -inf; their weights are 0
  const float m = m_run == -INFINITY ? 0.0f : m_run;
  return half_weights<VI8, MASKED>(acc, key0, c, weight_bias<QF>(c, m), pscale, nvalid, hh, pw);
}

// Fast-path acceptance: every lane's partial row sum is finite and at most
// kFastSum.  With m_run = -inf (no step yet) the weights are +inf and fail.
__device__ __forceinline__ bool fast_ok(float psum) { return __ballot(!(psum <= kFastSum)) == 0; }

// Per-lane LDS offsets of the tile readers (their layout terms depend only on
// the lane): k[x], the K operand of k-step x (row n, bytes 32x + 16hh: 16
// int8 or 8 bf16 channels); v[c], the V^T operand for output block c (rows
// hh*4 + j16/4 (+8), bytes 64c + (g16&1)*32 + (j16&3)*8 of the row).
template <int D, int KB>
struct LaneOffsets {
  static constexpr int KS = KB * D / 32;   // QK k-steps per half
  int k[KS];
  int v[D / 32];
};

// O^T += V^T.P^T for one 32-key half (two k-steps of 16 keys).
template <int D, int KB>
__device__ __forceinline__ void half_pv(const uint8_t* vbuf, int key0, const uint32_t (&pw)[8], v16f (&O)[D / 32],
                                        const LaneOffsets<D, KB>& lo);

// One weight pair (scores 2e, 2e+1 of a half) on the fast path: two FMAs, two
// exp2, one bf16 pack and the row-sum update.
template <bool VI8, class Acc>
__device__ __forceinline__ void weight_pair(const Acc& acc, int e, float c, float b, float pscale, float& psum,
                                            uint32_t (&pw)[8]) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(score_f(acc, 2 * e), c, b));
  const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(score_f(acc, 2 * e + 1), c, b));
  v2bf pk;
  if (VI8) {
    psum += p0 + p1;
    pk = (v2bf){(__bf16)(p0 * pscale), (__bf16)(p1 * pscale)};
  } else {
    pk = (v2bf){(__bf16)p0, (__bf16)p1};
    psum = __builtin_amdgcn_fdot2_f32_bf16(pk, (v2bf){(__bf16)1.0f, (__bf16)1.0f}, psum, false);
  }
  pw[e] = __builtin_bit_cast(uint32_t, pk);
}

// V^T operand of PV MFMA i (k-step i / NS of the half, output block i % NS).
template <int D, int KB>
__device__ __forceinline__ v8bf v_frag(const uint8_t* vbuf, int key0, int i, const LaneOffsets<D, KB>& lo) {
  using L = FwdLds<D>;
  constexpr int NS = D / 32;
  const uint8_t* p0 = vbuf + lo.v[i % NS] + (key0 + (i / NS) * 16) * L::VROW;
  return cat8(tr16(p0), tr16(p0 + 8 * L::VROW));
}

template <int D>
__device__ __forceinline__ v8bf p_frag(const uint32_t (&pw)[8], int i) {
  constexpr int NS = D / 32;
  const int k2 = i / NS;
  const v4i pwv = (v4i){(int)pw[k2 * 4], (int)pw[k2 * 4 + 1], (int)pw[k2 * 4 + 2], (int)pw[k2 * 4 + 3]};
  return __builtin_bit_cast(v8bf, pwv);
}

template <int D, int KB>
__device__ __forceinline__ void half_pv(const uint8_t* vbuf, int key0, const uint32_t (&pw)[8], v16f (&O)[D / 32],
                                        const LaneOffsets<D, KB>& lo) {
  constexpr int NS = D / 32;
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i)
    O[i % NS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag<D, KB>(vbuf, key0, i, lo), p_frag<D>(pw, i), O[i % NS],
                                                        0, 0, 0);
}

// The query fragment, the B operand of S^T = K.Q^T: lane (n, hh) holds query
// row n of its wave, channels 32s + 16hh .. +15 (int8) or 16s + 8hh .. +7
// (bf16) of k-step s.
template <int D, bool QF>
struct QFrag {
  v4i q[D / 32];
};
template <int D>
struct QFrag<D, true> {
  v8bf q[D / 16];
};

// One QK^T k-step: acc (+)= K_tile_rows . Q^T over the step's channels.
template <int D>
__device__ __forceinline__ v16i qk_mfma(v4i kop, const QFrag<D, false>& qf, int x, const v16i& acc) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, qf.q[x], acc, 0, 0, 0);
}
template <int D>
__device__ __forceinline__ v16f qk_mfma(v4i kop, const QFrag<D, true>& qf, int x, const v16f& acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, kop), qf.q[x], acc, 0, 0, 0);
}

// The exact 64-key tiles, as a software pipeline over 32-key halves.
//   S^T = K.Q^T on v_mfma_i32_32x32x32_i8 (exact int32); in a half the lane
//   holds query row n and keys (i/4)*8 + hh*4 + i%4 of it.
//   c = a_i * b_j * sm_scale * log2(e); weights p = exp2(S*c - m_run).
//   Each half is its own online-softmax step.  It first computes its weights
//   against m_run as it stands and keeps them when every lane's partial row
//   sum is finite and at most kFastSum; otherwise (the first step, a jump in
//   the scores) the exact step recomputes them after moving m_run.
//   The row sum adds the bf16-rounded p (v_dot2 with (1,1)), i.e. exactly the
//   weights the PV product uses.
//   O^T += V^T.P^T on v_mfma_f32_32x32x16_bf16, V^T via ds_read_b64_tr_b16.
// A wave issues in order and its weights are VALU work that can only overlap
// matrix-core work it issues in between, so step h of the pipeline puts the
// QK^T product of half h+1 and the PV product of half h-1 (12 MFMAs for
// d = 128) on the matrix cores and computes the 8 weight pairs of half h in
// their shadow, one MFMA and at most one pair per fixed scheduling segment.

template <bool B>
struct Parity {
  static constexpr bool value = B;
};

// MFMA m of a step with NQ QK MFMAs and NP PV MFMAs: QK and PV alternate
// while both are left (QK first, so the next scores are ready early).
template <int NQ, int NP>
__device__ constexpr bool step_is_qk(int m) {
  return NP == 0 || (NQ > 0 && m < 2 * NQ && m % 2 == 0);
}
template <int NQ, int NP>
__device__ constexpr int step_index(int m) {
  return (NQ == 0 || NP == 0) ? m : (m < 2 * NQ ? m / 2 : m - NQ);
}

// One pipeline step.  kh: the K half whose scores go to s_next (DO_QK);
// vh: the V half (32 rows) that p_prev weighs (DO_PV); s_cur: the scores
// whose weights go to p_cur (DO_W), with their row-sum part added to l_run
// after the fast-path check.  The copy pieces [P0, P1) of cp are issued in
// between, piece P0 + k in segment k.
template <int D, bool QF, bool VI8, bool DO_QK, bool DO_PV, bool DO_W, int P0, int P1>
__device__ __forceinline__ void pipe_step(const uint8_t* kh, const uint8_t* vh, const QFrag<D, QF>& qf,
                                          const SAcc<QF>& seed, SAcc<QF>& s_next, const SAcc<QF>& s_cur,
                                          const uint32_t (&p_prev)[8], uint32_t (&p_cur)[8], v16f (&O)[D / 32],
                                          float& m_run, float& l_run, float c, float pscale,
                                          const LaneOffsets<D, QF ? 2 : 1>& lo, int hh,
                                          const TileCopy<D, QF ? 2 : 1, VI8>& cp) {
  constexpr int NS = D / 32, KS = LaneOffsets<D, QF ? 2 : 1>::KS;
  constexpr int NQ = DO_QK ? KS : 0, NP = DO_PV ? 2 * NS : 0, M = NQ + NP, NC = P1 - P0;
  static_assert(M > 0, "a step issues matrix work");
  // A operands, loaded two MFMAs ahead (K rows: 16 int8 channels; V^T: 8 bf16)
  v4i op[M];
  auto load = [&](int m) {
    const int x = step_index<NQ, NP>(m);
    if (step_is_qk<NQ, NP>(m)) op[m] = *reinterpret_cast<const v4i*>(kh + lo.k[x]);
    else op[m] = __builtin_bit_cast(v4i, v_frag<D, QF ? 2 : 1>(vh, 0, x, lo));
  };
  float ps = 0.0f;
  const float b = weight_bias<QF>(c, m_run);
  load(0);
  if (M > 1) load(1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int x = step_index<NQ, NP>(m);
    if (step_is_qk<NQ, NP>(m))
      s_next = qk_mfma<D>(op[m], qf, x, x == 0 ? seed : s_next);
    else
      O[x % NS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, op[m]), p_frag<D>(p_prev, x),
                                                          O[x % NS], 0, 0, 0);
    if (m + 2 < M) load(m + 2);
    if (DO_W) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e * M / 8 == m) weight_pair<VI8>(s_cur, e, c, b, pscale, ps, p_cur);
    }
    static_assert(NC <= M, "at most one copy piece per scheduling segment");
#pragma unroll
    for (int k = 0; k < NC; ++k)
      if (k == m) cp.piece(P0 + k);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (DO_W) {
    if (!fast_ok(ps)) ps = half_exact<NS, VI8, false, QF>(s_cur, 0, c, pscale, kTile, hh, O, m_run, l_run, p_cur);
    l_run += ps;
  }
}

// The tile holding the end of a segment's valid keys (keys >= nvalid drop),
// done on its own with the exact step for both halves.
template <int D, bool QF, bool VI8>
__device__ __forceinline__ void masked_tile(const uint8_t* kbuf, const uint8_t* vbuf, const QFrag<D, QF>& qf,
                                            const SAcc<QF>& seed, v16f (&O)[D / 32], float& m_run, float& l_run,
                                            float c, float pscale, int nvalid, const LaneOffsets<D, QF ? 2 : 1>& lo,
                                            int hh) {
  constexpr int KB = QF ? 2 : 1;
  using L = FwdLds<D, KB>;
  constexpr int NS = D / 32, KS = LaneOffsets<D, KB>::KS;
  SAcc<QF> acc0 = seed, acc1 = seed;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    acc0 = qk_mfma<D>(*reinterpret_cast<const v4i*>(kbuf + lo.k[s]), qf, s, acc0);
    acc1 = qk_mfma<D>(*reinterpret_cast<const v4i*>(kbuf + 32 * L::KROW + lo.k[s]), qf, s, acc1);
  }
  uint32_t pw0[8], pw1[8];
  l_run += half_exact<NS, VI8, true, QF>(acc0, 0, c, pscale, nvalid, hh, O, m_run, l_run, pw0);
  half_pv<D, KB>(vbuf, 0, pw0, O, lo);
  l_run += half_exact<NS, VI8, true, QF>(acc1, 32, c, pscale, nvalid, hh, O, m_run, l_run, pw1);
  half_pv<D, KB>(vbuf, 32, pw1, O, lo);
}


}  // namespace

// QF: the exact tiles' QK^T on bf16 Q/K (fp32 scores) instead of the INT8
// codes; routing, centroids and everything after the scores are shared.
template <int D, bool QF, bool VI8, bool OBF16>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  constexpr int KB = QF ? 2 : 1;   // bytes per K element
  using L = FwdLds<D, KB>;
  constexpr int NS = D / 32;       // 32-channel output blocks
  constexpr int KS = LaneOffsets<D, KB>::KS;
  static_assert(!(QF && VI8), "the floating path takes bf16 V");
  // Two K and two V stages as separate LDS objects, so the compiler can see
  // that reading one stage does not depend on the direct loads into another.
  __shared__ __attribute__((aligned(16))) uint8_t kst0[L::KST];
  __shared__ __attribute__((aligned(16))) uint8_t kst1[L::KST];
  __shared__ __attribute__((aligned(16))) uint8_t vst0[L::VST];
  __shared__ __attribute__((aligned(16))) uint8_t vst1[L::VST];
  __shared__ uint16_t elist[2 * kWin];
  __shared__ uint16_t clist[kWin];
  __shared__ int plist[kMaxSegments], pvalid[kMaxSegments];
  __shared__ float bias[32];
  __shared__ int cnts[3];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  __builtin_assume(wave >= 0 && wave < 4);
  const int n = lane & 31, hh = lane >> 5;
  // per-lane LDS offsets of the tile readers (see LaneOffsets)
  LaneOffsets<D, KB> lo;
  {
    const int vq = hh * 4 + ((lane & 15) >> 2);
#pragma unroll
    for (int x = 0; x < KS; ++x) lo.k[x] = opaque(L::k_off(n, 32 * x + 16 * hh));
#pragma unroll
    for (int x = 0; x < NS; ++x) lo.v[x] = opaque(L::v_off(vq, 64 * x + ((lane >> 4) & 1) * 32 + (lane & 3) * 8));
  }

  // XCD-aware block order: hardware id b runs on XCD b % 8; give each XCD a
  // contiguous range of (head, query block) work items.
  const int nwg = gridDim.x;
  int bid = blockIdx.x;
  if ((nwg & 7) == 0) bid = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int i = bid % a.nQB;
  const int64_t bh = bid / a.nQB;
  const int nKS = QF ? 1 : a.Lkv / a.k_scale_rows;
  const int nVS = VI8 ? a.Lv / a.v_scale_rows : 1;
  const int tpb = a.kblock / kTile;   // 64-key tiles per key block

  // Q fragment (B operand of S^T = K.Q^T), see QFrag.
  const int qrow = i * kQBlock + wave * 32 + n;
  QFrag<D, QF> qf;
  if constexpr (QF) {
    const uint16_t* qp = a.qb + (bh * a.Lq + qrow) * D + hh * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf.q[s] = *reinterpret_cast<const v8bf*>(qp + s * 16);
  } else {
    const int8_t* qp = a.q + (bh * a.Lq + qrow) * D + hh * 16;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf.q[s] = *reinterpret_cast<const v4i*>(qp + s * 32);
  }
  // logit scale: c = qc * (K block scale) for the INT8 scores, qc for fp32 ones
  const float qc = QF ? a.sm_log2 : a.q_scale[bh * a.nQB + i] * a.sm_log2;

  // Initial value of the score accumulators: zero for fp32 scores; for the
  // INT8 ones the bit pattern kMagicI, built once (the empty asm keeps it in
  // registers instead of re-creating it per tile).
  SAcc<QF> seed;
  if constexpr (QF) {
    seed = (v16f){};
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) seed[e] = kMagicI;
    asm volatile("" : "+v"(seed));
  }
  v16f O[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) O[c] = (v16f){};
  float m_run = -INFINITY, l_run = 0.0f;
  const uint8_t* mrow = a.map + (bh * a.nQB + i) * a.nKB;
  const uint8_t* kbase = QF ? reinterpret_cast<const uint8_t*>(a.kb + bh * a.Lkv * D)
                            : reinterpret_cast<const uint8_t*>(a.k + bh * a.Lkv * D);
  const int8_t* v8base = static_cast<const int8_t*>(a.v) + bh * a.Lv * D;
  const uint8_t* v16base = static_cast<const uint8_t*>(a.v) + bh * a.Lv * D * 2;
  // buffer resources over this head's K and bf16 V (the tile copies); the
  // per-head sizes fit 32 bits (checked when the call is validated)
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(kbase, (uint32_t)((int64_t)a.Lkv * D * KB));
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(v16base, VI8 ? 0u : (uint32_t)((int64_t)a.Lv * D * 2));
  VRegs<D> vr;
  const DmaPlan<D, KB> plan = make_dma_plan<D, KB>(wave, lane);

  for (int w0 = 0; w0 < a.nKB; w0 += kWin) {
    const int wend = min(a.nKB, w0 + kWin);
    __syncthreads();
    if (wave == 0) {
      // Full exact tiles go to elist.  A tile holding the end of a segment's
      // valid keys (the valid keys of a block are a prefix of it) goes to
      // plist with its valid count: it needs masking and is done after the
      // pipelined loop.  Tiles without valid keys are skipped.
      int nE = 0, nC = 0, nP = 0;
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      for (int c0 = w0; c0 < wend; c0 += 64) {
        const int j = c0 + lane;
        const int st = j < wend ? mrow[j] : 0;
        const bool isE = st == 1, isC = st == 2 && a.G > 0;
        const int nv = isE ? a.lay.block_rows(j) : 0;
        const int nf = nv / kTile, pv = nv % kTile;   // full tiles, valid keys of the partial one
        const uint64_t b0 = __ballot(nf & 1), b1 = __ballot(nf & 2), bC = __ballot(isC), bP = __ballot(pv > 0);
        if (nf) {
          const int pos = nE + __popcll(b0 & lt) + 2 * __popcll(b1 & lt);
          for (int sub = 0; sub < nf; ++sub) elist[pos + sub] = (uint16_t)((j - w0) * tpb + sub);
        }
        if (pv > 0) {
          const int pos = nP + __popcll(bP & lt);
          if (pos < kMaxSegments) {
            plist[pos] = j * tpb + nf;
            pvalid[pos] = pv;
          }
        }
        if (isC) clist[nC + __popcll(bC & lt)] = (uint16_t)(j - w0);
        nE += __popcll(b0) + 2 * __popcll(b1);
        nC += __popcll(bC);
        nP += __popcll(bP);
      }
      if (lane == 0) {
        cnts[0] = nE;
        cnts[1] = nC;
        cnts[2] = min(nP, kMaxSegments);
      }
    }
    __syncthreads();
    const int nE = cnts[0], nC = cnts[1], nP = cnts[2];

    // ---------------- exact 64-key tiles, software pipeline ----------------
    // Tile T's halves are pipeline steps 2T and 2T+1 (see pipe_step).  K
    // stages hold tiles by parity and V stages too, one tile behind: between
    // the barriers that open tile iterations T and T+1 the waves read K of
    // tile T+1 and V of tile T while the copies of K of tile T+2 and V of tile
    // T+1 fill the other two stages.  When no tile T+2 exists the K copy
    // repeats tile T+1 into the free stage, which nothing reads.
    // Registers: scores of even halves sA, odd halves sB; weights pA / pB.
    if (nE > 0) {
      // Every copy piece goes into a tile's first step, one per scheduling
      // segment from its start: the copies then have the rest of the tile to
      // land before the next barrier waits for them (measured faster than
      // spreading them over both steps or issuing two per segment).
      constexpr int PH = TileCopy<D, KB, VI8>::PIECES;   // copy pieces in a tile's first step
      constexpr int PN = TileCopy<D, KB, VI8>::PIECES;
      TileInfo t0 = fetch_tile<QF, VI8>(a, bh, w0 * tpb + __builtin_amdgcn_readfirstlane(elist[0]), nKS, nVS);
      TileInfo t1 = nE > 1 ? fetch_tile<QF, VI8>(a, bh, w0 * tpb + __builtin_amdgcn_readfirstlane(elist[1]), nKS, nVS) : t0;
      // list entry of tile T + 2, read one iteration before it is needed so
      // the top of an iteration does not wait for an LDS read
      int next_entry = elist[min(2, nE - 1)];
      if (VI8) load_v_int8<D>(v8base + (int64_t)t0.vrow0() * D, vr, tid);
      tile_copy<D, KB, VI8>(t0, t0, kst0, vst0, krs, vrs, plan, wave).all();
      tile_copy<D, KB, VI8>(t1, t1, kst1, vst1, krs, vrs, plan, wave).all_k();
      if (VI8) store_v_int8<D>(vst0, vr, tid);
      copies_done_barrier();
      SAcc<QF> sA, sB;
      uint32_t pA[8], pB[8];
      // step 0: scores of half 0 first, then half 1's with half 0's weights
      pipe_step<D, QF, VI8, true, false, false, 0, 0>(kst0, vst0, qf, seed, sA, seed, pB, pA, O, m_run, l_run, 0.0f, 0.0f,
                                                  lo, hh, TileCopy<D, KB, VI8>{});
      pipe_step<D, QF, VI8, true, false, true, 0, 0>(kst0 + 32 * L::KROW, vst0, qf, seed, sB, sA, pB, pA, O, m_run,
                                                 l_run, qc * t0.kscale, t0.pscale, lo, hh,
                                                 TileCopy<D, KB, VI8>{});
      // Tile iteration T (T + 1 < nE), between the barrier that opens it and
      // the next one: steps 2T+1 and 2T+2.  ODD is T's parity, which picks the
      // stages at compile time.
      auto tile_iter = [&](auto odd, int T) {
        constexpr bool ODD = decltype(odd)::value;
        uint8_t* const krd = ODD ? kst0 : kst1;   // K of tile T+1
        uint8_t* const vrd = ODD ? vst1 : vst0;   // V of tile T
        uint8_t* const kwr = ODD ? kst1 : kst0;   // K of tile T+2 goes here
        uint8_t* const vwr = ODD ? vst0 : vst1;   // V of tile T+1 goes here
        copies_done_barrier();
        const TileInfo t2 =
            T + 2 < nE ? fetch_tile<QF, VI8>(a, bh, w0 * tpb + __builtin_amdgcn_readfirstlane(next_entry), nKS, nVS)
                       : t1;
        next_entry = elist[min(T + 3, nE - 1)];
        if (VI8) load_v_int8<D>(v8base + (int64_t)t1.vrow0() * D, vr, tid);
        const TileCopy<D, KB, VI8> cp = tile_copy<D, KB, VI8>(t2, t1, kwr, vwr, krs, vrs, plan, wave);
        pipe_step<D, QF, VI8, true, true, true, 0, PH>(krd, vrd, qf, seed, sA, sB, pA, pB, O, m_run, l_run,
                                                   qc * t0.kscale, t0.pscale, lo, hh, cp);
        pipe_step<D, QF, VI8, true, true, true, PH, PN>(krd + 32 * L::KROW, vrd + 32 * L::VROW, qf, seed, sB, sA, pB,
                                                    pA, O, m_run, l_run, qc * t1.kscale, t1.pscale, lo, hh,
                                                    cp);
        if (VI8) store_v_int8<D>(vwr, vr, tid);
        t0 = t1;
        t1 = t2;
      };
      int T = 0;
      for (; T + 2 < nE; T += 2) {
        tile_iter(Parity<false>{}, T);
        tile_iter(Parity<true>{}, T + 1);
      }
      if (T + 1 < nE) tile_iter(Parity<false>{}, T++);
      // last tile T: PV of its first half with the weights of its second, then
      // PV of the second (no copies are in flight, so the stage can be picked
      // at run time)
      copies_done_barrier();
      const uint8_t* vl = (T & 1) ? vst1 : vst0;
      pipe_step<D, QF, VI8, false, true, true, 0, 0>(kst0, vl, qf, seed, sA, sB, pA, pB, O, m_run, l_run,
                                                 qc * t0.kscale, t0.pscale, lo, hh, TileCopy<D, KB, VI8>{});
      half_pv<D, KB>(vl, 32, pB, O, lo);
    }
    copies_done_barrier();                       // stages free again
    for (int pi = 0; pi < nP; ++pi) {            // tiles with the end of a segment's valid keys
      const TileInfo t = fetch_tile<QF, VI8>(a, bh, plist[pi], nKS, nVS);
      const int nvalid = pvalid[pi];
      if (VI8) load_v_int8<D>(v8base + (int64_t)t.vrow0() * D, vr, tid);
      tile_copy<D, KB, VI8>(t, t, kst0, vst0, krs, vrs, plan, wave).all();
      if (VI8) store_v_int8<D>(vst0, vr, tid);
      copies_done_barrier();
      // Keys at or past nvalid get weight 0, but their V rows are padding and
      // may hold anything (NaN, Inf): clear them so that 0 * V stays 0 in the
      // PV product.
      for (int u = tid; u < (kTile - nvalid) * (L::VROW / 16); u += 256) {
        const int r = nvalid + u / (L::VROW / 16), x = (u % (L::VROW / 16)) * 16;
        *reinterpret_cast<v4i*>(vst0 + L::v_off(r, x)) = (v4i){0, 0, 0, 0};
      }
      __syncthreads();
      masked_tile<D, QF, VI8>(kst0, vst0, qf, seed, O, m_run, l_run, qc * t.kscale, t.pscale, nvalid, lo, hh);
      __syncthreads();
    }

    // ---------------- centroid columns, 32 at a time ----------------
    // Staging: 8 threads per column, each converting CE consecutive 4-channel
    // pieces of one centroid to bf16 hi+lo pairs.  Column (key block j, group
    // g) is row j*G + g of this head's centroids (G is 1 or 2 here).  The rows
    // are loaded whatever the count; a count of 0 only selects zeros.
    const int ncols = nC * a.G;
    constexpr int CE = D / 32;
    const int64_t chead = bh * a.nKB * a.G;
    const float* kch = a.kc + chead * D;
    const float* vch = a.vc + chead * D;
    const float* cnh = a.cnt + chead;
    for (int c0 = 0; c0 < ncols; c0 += 32) {
      {
        // INT8 V: thread roles formed again from the thread index here; hoisted
        // out of the window loop, the per-thread addresses would live across
        // the tile loop next to the V staging registers (and be spilled)
        const int st = VI8 ? opaque(tid) : tid, col = st >> 3, q = st & 7;
        const int ent = c0 + col, be = a.G == 2 ? ent >> 1 : ent, g = a.G == 2 ? ent & 1 : 0;
        float cn = 0.0f;
        float4 kv[CE], vv[CE];
#pragma unroll
        for (int e = 0; e < CE; ++e) kv[e] = vv[e] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (be < nC) {
          const int cl = (w0 + clist[be]) * a.G + g;
          cn = cnh[cl];
#pragma unroll
          for (int e = 0; e < CE; ++e) {
            kv[e] = reinterpret_cast<const float4*>(kch + cl * D)[q * CE + e];
            vv[e] = reinterpret_cast<const float4*>(vch + cl * D)[q * CE + e];
          }
        }
        const bool has = cn > 0.0f;
#pragma unroll
        for (int e = 0; e < CE; ++e) {
          const int c4 = q * CE + e;
          const float kf[4] = {kv[e].x, kv[e].y, kv[e].z, kv[e].w}, vf[4] = {vv[e].x, vv[e].y, vv[e].z, vv[e].w};
          v4bf khi, klo, vhi, vlo;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float kx = has ? kf[e2] : 0.0f, vx = has ? vf[e2] : 0.0f;
            khi[e2] = (__bf16)kx;
            klo[e2] = (__bf16)(kx - (float)khi[e2]);
            vhi[e2] = (__bf16)vx;
            vlo[e2] = (__bf16)(vx - (float)vhi[e2]);
          }
          *reinterpret_cast<v4bf*>(vst0 + L::kc_off(col, c4 * 8)) = khi;
          *reinterpret_cast<v4bf*>(vst0 + L::KCL_OFF + L::kc_off(col, c4 * 8)) = klo;
          *reinterpret_cast<v4bf*>(vst1 + L::v_off(col, c4 * 8)) = vhi;
          *reinterpret_cast<v4bf*>(vst1 + L::VCL_OFF + L::v_off(col, c4 * 8)) = vlo;
        }
        if (q == 0) bias[col] = has ? __log2f(cn) : -INFINITY;
      }
      __syncthreads();
      // q . K-bar on bf16 MFMA: the INT8 query codes (exact in bf16; the query
      // scale is in qc) or the bf16 query, against the hi and lo parts
      v16f acc = (v16f){};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        v8bf qb;
        int ch;   // first channel of this lane's 8 in k-step s
        if constexpr (QF) {
          qb = qf.q[s];
          ch = s * 16 + hh * 8;
        } else {
          v4i qv = qf.q[s / 2];
          // INT8 V: converted here each batch; hoisted out of the loops, the
          // bf16 query would stay live across the tile loop and be spilled
          if (VI8) asm volatile("" : "+v"(qv));
          qb = i8x8_to_bf16(qv[2 * (s % 2)], qv[2 * (s % 2) + 1]);
          ch = (s / 2) * 32 + hh * 16 + (s % 2) * 8;
        }
        const int off = L::kc_off(n, ch * 2);
        const v8bf khi = *reinterpret_cast<const v8bf*>(vst0 + off);
        const v8bf klo = *reinterpret_cast<const v8bf*>(vst0 + L::KCL_OFF + off);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi, qb, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo, qb, acc, 0, 0, 0);
      }
      float x[16];
      float mx = -INFINITY;
#pragma unroll
      for (int e2 = 0; e2 < 16; ++e2) {
        const int col = (e2 / 4) * 8 + hh * 4 + (e2 % 4);
        x[e2] = __builtin_fmaf(acc[e2], qc, bias[col]);
        mx = fmaxf(mx, x[e2]);
      }
      mx = pair_max(mx);
      maybe_rescale<NS>(mx, m_run, l_run, O);
      const float msub = m_run == -INFINITY ? 0.0f : m_run;
      float psum = 0.0f;
#pragma unroll
      for (int e2 = 0; e2 < 16; ++e2) {
        x[e2] = __builtin_amdgcn_exp2f(x[e2] - msub);
        psum += x[e2];
      }
      l_run += psum;
      const int g16 = lane >> 4, j16 = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8bf pf;
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) pf[e2] = (__bf16)x[ks * 8 + e2];
        const int krow = ks * 16 + hh * 4 + (j16 >> 2);
#pragma unroll
        for (int cb = 0; cb < NS; ++cb) {
          const int col = cb * 32 + (g16 & 1) * 16 + 4 * (j16 & 3);
          const int o0 = L::v_off(krow, col * 2), o8 = L::v_off(krow + 8, col * 2);
          const v8bf vh = cat8(tr16(vst1 + o0), tr16(vst1 + o8));
          const v8bf vl = cat8(tr16(vst1 + L::VCL_OFF + o0), tr16(vst1 + L::VCL_OFF + o8));
          O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, pf, O[cb], 0, 0, 0);
          O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl, pf, O[cb], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }

  // ---------------- finalize ----------------
  // Padded rows and rows with nothing to attend are written as 0 by a select
  // (not by a zero factor, which would keep a NaN from a padded query row).
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  // the output row, formed again from the thread index (kept live across the
  // tile loop instead, it would be spilled)
  const int qrow_out = i * kQBlock + ((opaque(tid) >> 6) << 5) + n;   // wave * 32 + n
  const bool row_ok = qrow_out < a.lq_valid && l_tot > 0.0f;
  const float inv = row_ok ? 1.0f / l_tot : 0.0f;
#pragma unroll
  for (int cb = 0; cb < NS; ++cb) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int ch = cb * 32 + gq * 8 + hh * 4;
      const int64_t o = (bh * a.Lq + qrow_out) * D + ch;
      if (OBF16) {
        v4bf r;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) r[e2] = (__bf16)(row_ok ? O[cb][gq * 4 + e2] * inv : 0.0f);
        *reinterpret_cast<v4bf*>(static_cast<uint16_t*>(a.out) + o) = r;
      } else {
        float x[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) x[e2] = row_ok ? O[cb][gq * 4 + e2] * inv : 0.0f;
        const float4 r = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o) = r;
      }
    }
  }
  if (a.lse && hh == 0)
    a.lse[bh * a.Lq + qrow_out] = row_ok ? (m_run + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
}

template <int D, bool VI8>
static hipError_t launch_fwd_dv(const FwdArgs& a, hipStream_t st) {
  dim3 grid(a.B * a.H * a.nQB);
  if (a.out_bf16) fwd_kernel<D, false, VI8, true><<<grid, 256, 0, st>>>(a);
  else fwd_kernel<D, false, VI8, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  if (a.d == 64) return a.v_int8 ? launch_fwd_dv<64, true>(a, st) : launch_fwd_dv<64, false>(a, st);
  return a.v_int8 ? launch_fwd_dv<128, true>(a, st) : launch_fwd_dv<128, false>(a, st);
}

// The floating path: the same kernel with bf16 Q/K (and bf16 V).
template <int D>
static hipError_t launch_fwd_float_d(const FwdArgs& a, hipStream_t st) {
  dim3 grid(a.B * a.H * a.nQB);
  if (a.out_bf16) fwd_kernel<D, true, false, true><<<grid, 256, 0, st>>>(a);
  else fwd_kernel<D, true, false, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd_float(const FwdFloatArgs& f, hipStream_t st) {
  FwdArgs a{};
  a.qb = f.q;
  a.kb = f.k;
  a.v = f.v;
  a.v_block_src = f.v_block_src;
  a.map = f.map;
  a.kc = f.kc;
  a.vc = f.vc;
  a.cnt = f.cnt;
  a.out = f.out;
  a.lse = f.lse;
  a.B = f.B; a.H = f.H; a.Lq = f.Lq; a.Lkv = f.Lkv; a.Lv = f.Lv; a.d = f.d;
  a.lq_valid = f.lq_valid; a.lkv_valid = f.lkv_valid;
  a.nQB = f.nQB; a.nKB = f.nKB; a.kblock = f.kblock; a.G = f.G;
  a.k_scale_rows = kTile;   // unused on this path (no K scales); kept non-zero
  a.v_scale_rows = kTile;
  a.ks_shift = a.vs_shift = 6;
  a.lay = f.lay;
  a.v_int8 = false;
  a.out_bf16 = f.out_bf16;
  a.sm_log2 = f.sm_log2;
  return f.d == 64 ? launch_fwd_float_d<64>(a, st) : launch_fwd_float_d<128>(a, st);
}

}  // namespace sa
