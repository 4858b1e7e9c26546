// attention.hip — the persistent split-K attention kernel (Split-K stage).
//
// "Triton-TLE rewrite of Tencent HPC-Ops Attention", §1.2: persistent
// workgroups walk the task map; per KV tile they compute QK, the mask, an fp32
// online softmax and PV, and emit either the final output (a Q-block owned by
// one worker) or a partial output + LSE (split Q-blocks, merged by Combine).
// The same kernel serves decode rows and prefill chunks in one launch
// ("Chunked Prefill kernel optimisation: Triton hybrid attention": one fused
// kernel for a hybrid batch) and reads its work from GPU metadata with a grid
// of fixed size ("vLLM Triton Attention Backend Deep Dive", §3, persistent
// kernels).
//
// gfx950 design (not the Hopper TMA / WGMMA / warp-specialised design of the
// pages): every product runs on 16x16 MFMA in the transposed form
//     S^T = K Q^T   (M = 16 keys, N = 16 query rows, K = head dims)
//     O^T = V^T P^T (M = 16 dims, N = 16 query rows, K = keys)
// so a lane always owns one query row: the 16x16 accumulator layout gives lane
// l the column l % 16 and rows 4 (l / 16) + j.  The row max and row sum of the
// online softmax are then in-lane plus two cross-lane steps, the rescale of
// the O accumulator needs no shuffle, and the P operand of the PV product is
// built from the lane's own S values (the key order inside a PV K-step is
// chosen to match; V is gathered in that same order).  This is the small-M
// idea of the Triton-TLE page (§3.1, KV tile on the MFMA M side, query heads
// on N) carried through both products.
//
// Two Q-block shapes:
//  * small (q_len * G <= 16 rows, decode / MTP): memory-bound.  The four
//    waves of a workgroup take disjoint runs of the worker's units and load
//    K and V straight from HBM into MFMA operand registers (K rows are already
//    k-contiguous; V rows are transposed in registers with byte permutes).
//    The four partial states are merged through LDS at the end.
//  * large (128 rows = 128 / G tokens x G heads, prefill): compute-bound.
//    Each wave owns 32 rows; K and V tiles are staged once per workgroup into
//    LDS in MFMA-operand order and double-buffered.
// Block-sparse prefill compacts the active tiles of a Q-block with a 64-lane
// ballot + mbcnt prefix into an LDS list ("Triton-TLE ...", §2.1).
#include <atomic>
#include <type_traits>

#include "combine_core.h"
#include "pa_device.h"

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

template <int KIND, int D>
struct Cfg {
  static constexpr int MD = D / 16;                                  // O^T M-blocks; V elements per lane per row load
  static constexpr int KSQ = KIND == KIND_F32 ? D / 4 : D / 32;      // QK K-steps
  static constexpr int ELT = KIND == KIND_F32 ? 4 : KIND == KIND_BF16 ? 2 : 1;
  static constexpr int K_TILE = 64 * D * ELT;                        // LDS bytes, K tile (operand order)
  static constexpr int V_TILE = 64 * D * (KIND == KIND_F32 ? 4 : 2);  // V staged as bf16 for fp8
  static constexpr int STAGE = K_TILE + V_TILE;
  static constexpr int MERGE = kWaves * kSmallMaxRows * (D + 2) * 4;  // small-path wave merge
  static constexpr int QOFF = (MERGE + 255) / 256 * 256;               // small-path Q operands
  static constexpr int QBYTES = KSQ * 64 * (KIND == KIND_F32 ? 4 : KIND == KIND_BF16 ? 16 : 8);
  // small_range: merge stash of 8 cut pieces (m, l, raw O per row) and tags
  static constexpr int STASH = (2 * kWaves) * (32 + 16 * D) * 4 + 2 * kWaves * 4;
  static constexpr int BODY0 = 2 * STAGE > QOFF + QBYTES ? 2 * STAGE : QOFF + QBYTES;
  static constexpr int LDS = (BODY0 > STASH ? BODY0 : STASH) + kMaskListCap * 2;
  // workgroups per compute unit: two (so that each SIMD runs two waves) where
  // half the LDS suffices, else one
  static constexpr int OCC = LDS <= 80 * 1024 ? 2 : 1;
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// bf16 or fp8, d = 128, one page per tile (the direct paths): the two V stages
// (bf16, row-major) are LDS arrays of their own (vstage), the rest stays in
// the dynamic block.  The compiler then knows that a DMA into one V stage
// cannot touch the transpose reads of the other and issues those reads
// without waiting for every DMA in flight.  fp8 V lands first in an 8 KiB
// staging block after the two K stages and is widened into the V stage.
// Small ranges keep four of their eight stash pieces in the V stages.
constexpr int kVStageBytes = 16384;
constexpr int kV8Bytes = 64 * 128;      // one fp8 V tile (d = 128)
template <int KIND, int D, bool FAST>
struct Lds {
  using C = Cfg<KIND, D>;
  static constexpr bool SPLIT_V = (KIND == KIND_BF16 || KIND == KIND_F8) && D == 128 && FAST;
  static constexpr int STASH_PIECES_DYN = SPLIT_V ? kWaves : 2 * kWaves;      // acc pieces in the dynamic block
  static constexpr int STASH_DYN = (2 * 2 * kWaves * 16 + STASH_PIECES_DYN * 16 * D) * 4 + 2 * kWaves * 4;
  static constexpr int KV_DYN = 2 * C::K_TILE + (KIND == KIND_F8 ? kV8Bytes : 0);   // K stages (+ fp8 V staging)
  static constexpr int BODY = SPLIT_V ? (KV_DYN > C::QOFF + C::QBYTES ? KV_DYN : C::QOFF + C::QBYTES)
                                      : C::BODY0;
  static constexpr int DYN = (BODY > STASH_DYN ? BODY : STASH_DYN) + kMaskListCap * 2;
  static constexpr int TOTAL = DYN + (SPLIT_V ? 2 * kVStageBytes : 0);
  static constexpr int OCC = TOTAL <= 80 * 1024 ? 2 : 1;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  // the lean bf16 build: three K stages and nothing else in the dynamic block
  // (with the two V stages exactly 80 KiB, so two workgroups share a CU)
  static constexpr int DYN_LEAN = KIND == KIND_BF16 ? 3 * C::K_TILE : DYN;
  static_assert(KIND != KIND_BF16 || !SPLIT_V || DYN_LEAN + 2 * kVStageBytes <= 80 * 1024, "lean LDS budget");
  static_assert(DYN_LEAN >= 256 * 40 + 4, "fused merge slots");
  static_assert(!SPLIT_V || 2 * 16 * D * 4 <= kVStageBytes, "two stash pieces per V stage");
};

template <bool ON>
__device__ __forceinline__ char* vstage(int i) {
  __shared__ __attribute__((aligned(16))) char v0[ON ? kVStageBytes : 16];
  __shared__ __attribute__((aligned(16))) char v1[ON ? kVStageBytes : 16];
  return i ? v1 : v0;
}

template <int KIND> struct QKOpT;
template <> struct QKOpT<KIND_F32> { using T = float; };
template <> struct QKOpT<KIND_BF16> { using T = bf16x8; };
template <> struct QKOpT<KIND_F8> { using T = long; };

__device__ __forceinline__ f32x4 mfma_qk(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_qk(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_qk(long a, long b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}
// fp8, d = 128: one 16x16x128 MFMA over the whole head dim.  A lane's four
// 16x16x32 K-step operands, concatenated, pair slot for slot with the Q row's
// four operands concatenated the same way, so the sum runs over all 128 dims.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ i32x8 cat4(long a0, long a1, long a2, long a3) {
  return i32x8{(int)a0, (int)(a0 >> 32), (int)a1, (int)(a1 >> 32), (int)a2, (int)(a2 >> 32), (int)a3, (int)(a3 >> 32)};
}
__device__ __forceinline__ f32x4 mfma_qk128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);   // E4M3 x E4M3, no block scales
}
__device__ __forceinline__ f32x4 mfma_pv(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};          // round to nearest even
  return __builtin_bit_cast(unsigned, v);
}

// Two E4M3FN bytes of w (bits 0-15, or 16-31 with HI) -> two bf16 in one
// word, exactly (every E4M3FN value is a bf16), by the hardware conversion
// at scale 1.  NaN codes stay NaN: they only occur in cache slots past a
// sequence's end, which are clamped away or zeroed before use.
template <bool HI = false>
__device__ __forceinline__ unsigned f8x2_to_bf16x2(unsigned w) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// ---------------------------------------------------------------------------
// addressing.  Every load address is valid: keys past the end of a sequence
// are clamped to its last key (their probability is exactly 0, so the finite
// data they bring contributes nothing), and a block-table entry outside
// [0, num_pages) is replaced by page 0 and reported in the error word.
// ---------------------------------------------------------------------------
struct SeqCtx {
  int b, g, ctx, t_lo;
  const int32_t* bt_row;
};

__device__ __forceinline__ int page_of(const KParams& p, const SeqCtx& s, int key) {
  const int idx = key >> p.page_shift;
  int page = idx < p.max_pages ? s.bt_row[idx] : -1;
  if ((unsigned)page >= (unsigned)p.num_pages) {
    p.hdr[H_ERROR] = E_PAGE;
    page = 0;
  }
  return page;
}

// The kernel's parameter block, read through the kernarg segment pointer (the
// block is the kernel's only argument, at offset 0).  Every use site takes its
// own opaque copy of the pointer, so a segment loads the parameters it needs
// (scalar loads) where it starts, instead of the whole persistent kernel
// holding every parameter in scalar registers from the first instruction.  The
// pointer itself exists only in the kernel (a called function would see null),
// so the kernel reads it once and hands the value down (kparams_at).
// A 64-bit value made wave-uniform.  The builtin returns a signed int, so each
// half goes through uint32_t before widening (no sign extension).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Segment functions are inlined into the kernel: measured faster than
// separate calls (whose callee-saved registers and call boundaries cost more
// than the separate register allocation gains).
#ifndef PA_SEGMENT_FN
#define PA_SEGMENT_FN __attribute__((always_inline))
#endif

__device__ __forceinline__ uint64_t kparams_addr() {
  return reinterpret_cast<uint64_t>(__builtin_amdgcn_kernarg_segment_ptr());
}
__device__ __forceinline__ const KParams& kparams_at(uint64_t v) {
  v = uniform_u64(v);
  asm volatile("" : "+s"(v));
  return *(const KParams*)(const __attribute__((address_space(4))) KParams*)v;
}

// Reductions over the four lanes n, n + 16, n + 32, n + 48 that share a query
// row, with the lane-swap instructions (no LDS round trip): the swap of a
// register with itself hands each lane both halves of the exchanged pair.
// max of two scores that are never NaN (masked ones are -inf): a plain
// v_max_f32, without the quieting copies fmaxf adds for operands the compiler
// cannot prove canonical (a cross-lane swap's results)
__device__ __forceinline__ float max_nonan(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_nonan(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float row_max4(float x) {
  const unsigned u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);      // lanes l & ~16, l | 16
  x = max_nonan(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned w = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);      // lanes l & ~32, l | 32
  return max_nonan(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
  const unsigned u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned w = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Values the whole wave shares, made explicit for the compiler (so addressing
// stays in scalar registers and buffer resources need no per-lane loop).
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const char* wave_uniform(const char* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// A parameter held in a scalar register from here on.  Parameters are
// invariant loads, so under register pressure the compiler would rather
// re-load one inside a loop than keep it; each such load is followed by a
// wait that also drains the loop's in-flight LDS reads.  The value an empty
// asm hands back cannot be re-loaded, only kept (or spilled to a lane).
__device__ __forceinline__ int held(int v) {
  v = __builtin_amdgcn_readfirstlane(v);
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ float held(float v) { return __int_as_float(held(__float_as_int(v))); }

// Loads at base + soff + voff: `base + soff` is wave-uniform (scalar), voff a
// 32-bit per-lane offset, so the address is a scalar base plus a VGPR offset
// when the compiler keeps the base in scalar registers.
//
// The 16-byte load is non-temporal: its users stream K/V rows that are read
// once (decode tiles), and not allocating them in the caches moved the bf16
// decode kernel from 5.05 to 5.35 TB/s (NHD) and 5.31 to 5.95 TB/s (HND) on
// MI355X.  The temporal 8-byte load serves the fp8 K rows of the per-kv-head
// paths (with 8-byte V rows also temporal, fp8 decode once ran 41% slower
// non-temporal; the V rows alone non-temporal are faster, see gload8nt).
#define PA_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ u32x4 gload16(const char* base, uint32_t voff, uint32_t soff) {
  return __builtin_nontemporal_load((const PA_GLOBAL u32x4*)(base + soff + voff));
}
__device__ __forceinline__ u32x2 gload8(const char* base, uint32_t voff, uint32_t soff) {
  return *(const PA_GLOBAL u32x2*)(base + soff + voff);
}
// temporal 16-byte load: the bf16 K rows of per-kv-head small Q-blocks
// (small_range and small_segment), where it measured faster on MI355X (MTP 4
// decode 2%, the hybrid batch 7%, a statically split 128K decode 9.5%; V
// stays non-temporal there: temporal V was 8% slower).  The sequence-Q-block
// path keeps its K rows non-temporal, bf16 and paired fp8 alike (temporal:
// bf16 1.8% slower on HND; fp8 2% slower at q_len 2 and on HND)
__device__ __forceinline__ u32x4 gload16t(const char* base, uint32_t voff, uint32_t soff) {
  return *(const PA_GLOBAL u32x4*)(base + soff + voff);
}
// non-temporal 8-byte load: fp8 V rows (d = 128) and bf16 V rows (d = 64)
// of decode, each read once; measured 8% faster than temporal for fp8 decode
// q_len 1 (NHD and HND) and 3% at q_len 4 on MI355X, with the fp8 K rows
// temporal beside them
__device__ __forceinline__ u32x2 gload8nt(const char* base, uint32_t voff, uint32_t soff) {
  return __builtin_nontemporal_load((const PA_GLOBAL u32x2*)(base + soff + voff));
}
__device__ __forceinline__ unsigned gload4(const char* base, uint32_t voff, uint32_t soff) {
  return *(const PA_GLOBAL unsigned*)(base + soff + voff);
}
// Direct HBM -> LDS through a buffer resource: every lane fetches 16 B at
// rsrc.base + soff + voff; the wave writes them lane-linearly (1 KiB) at the
// wave-uniform LDS address `dst`.  The base lives in scalar registers (a
// resource per tile) and the lane offset in a VGPR fixed for a segment, so a
// DMA costs no vector address arithmetic (a 64-bit global address per lane
// took two VALU instructions and read-backs per DMA).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base) {
  // raw buffer: no stride, a range past any offset used (offsets stay inside
  // one page of the cache), the gfx9 default data format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void bload16_lds(__amdgpu_buffer_rsrc_t rsrc, char* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

// Rows of one 64-key tile.  FAST (page_size >= 64): the tile lies in one page,
// so the page lookup and the row base are uniform (scalar) and each lane adds a
// 32-bit offset.  Otherwise every key looks up its own page.
template <int ELT, bool FAST>
struct Tile {
  const char* kb;       // FAST: the tile's first row (key J0, kv head g) in K and V
  const char* vb;
  int J0, nvalid;
  int page;             // FAST: physical page of the tile
  uint32_t kss, vss;   // bytes between consecutive keys of a page

  // FAST only: the page holding key J0 is already known
  __device__ __forceinline__ void init_at_page(const KParams& p, const SeqCtx& s, int tile, int page) {
    J0 = wave_uniform(tile) * kUnitKeys;
    nvalid = wave_uniform(min(kUnitKeys, s.ctx - J0));
    kss = (uint32_t)(p.k_ss * ELT);
    vss = (uint32_t)(p.v_ss * ELT);
    this->page = page;
    const int slot = J0 & (p.page_size - 1);
    kb = wave_uniform(reinterpret_cast<const char*>(p.k) +
                      ((int64_t)page * p.k_sp + (int64_t)slot * p.k_ss + (int64_t)s.g * p.k_sh) * ELT);
    vb = wave_uniform(reinterpret_cast<const char*>(p.v) +
                      ((int64_t)page * p.v_sp + (int64_t)slot * p.v_ss + (int64_t)s.g * p.v_sh) * ELT);
  }
  __device__ __forceinline__ void init(const KParams& p, const SeqCtx& s, int tile) {
    J0 = wave_uniform(tile) * kUnitKeys;
    nvalid = wave_uniform(min(kUnitKeys, s.ctx - J0));
    kss = (uint32_t)(p.k_ss * ELT);
    vss = (uint32_t)(p.v_ss * ELT);
    if constexpr (FAST) {
      page = page_of(p, s, J0);
      const int slot = J0 & (p.page_size - 1);
      kb = reinterpret_cast<const char*>(p.k) + ((int64_t)page * p.k_sp + (int64_t)slot * p.k_ss + (int64_t)s.g * p.k_sh) * ELT;
      vb = reinterpret_cast<const char*>(p.v) + ((int64_t)page * p.v_sp + (int64_t)slot * p.v_ss + (int64_t)s.g * p.v_sh) * ELT;
      kb = wave_uniform(kb);
      vb = wave_uniform(vb);
    }
  }
  __device__ __forceinline__ const char* krow(const KParams& p, const SeqCtx& s, int kt) const {
    const int kk = min(kt, nvalid - 1);
    if constexpr (FAST) {
      return kb + (uint32_t)kk * kss;
    } else {
      const int key = J0 + kk;
      const int page = page_of(p, s, key);
      return reinterpret_cast<const char*>(p.k) +
             ((int64_t)page * p.k_sp + (int64_t)(key & (p.page_size - 1)) * p.k_ss + (int64_t)s.g * p.k_sh) * ELT;
    }
  }
  __device__ __forceinline__ const char* vrow(const KParams& p, const SeqCtx& s, int kt) const {
    const int kk = min(kt, nvalid - 1);
    if constexpr (FAST) {
      return vb + (uint32_t)kk * vss;
    } else {
      const int key = J0 + kk;
      const int page = page_of(p, s, key);
      return reinterpret_cast<const char*>(p.v) +
             ((int64_t)page * p.v_sp + (int64_t)(key & (p.page_size - 1)) * p.v_ss + (int64_t)s.g * p.v_sh) * ELT;
    }
  }
};

// Scales of a tile whose physical page is known (page_size >= 64).
template <int KIND>
__device__ __forceinline__ float kscale_at_page(const KParams& p, const SeqCtx& s, int page, float* vsc) {
  if constexpr (KIND != KIND_F8) {
    *vsc = 1.f;
    return 1.f;
  } else {
    const int i = (p.scale_mode & 3) == 2 ? page * p.Hkv + s.g : 0;
    *vsc = p.v_scale[i];
    return p.k_scale[i];
  }
}

// fp8 K and V scales read once by a caller that runs many tiles, in
// per-tensor mode.  `valid` is false for per-(page, head) scales, which stay
// a per-tile load, and for bf16 and fp32 (scales of 1, no load).  Without it
// the two scale loads of every tile sit between the tile's K/V loads and its
// softmax, which then waits for them as well.
struct KvScales {
  float k, v;
  bool valid;
};
template <int KIND>
__device__ __forceinline__ KvScales kv_scales_hoisted(const KParams& p) {
  if constexpr (KIND != KIND_F8) return KvScales{1.f, 1.f, false};
  else {
    if ((p.scale_mode & 3) == 2) return KvScales{1.f, 1.f, false};
    return KvScales{p.k_scale[0], p.v_scale[0], true};
  }
}

// Q scale of one query row: per tensor, or per (query token, query head)
// from a [total_q, Hq] array.
template <int KIND>
__device__ __forceinline__ float qscale_of(const KParams& p, int tok, int head) {
  if constexpr (KIND != KIND_F8) return 1.f;
  else return (p.scale_mode & 4) ? p.q_scale[(int64_t)tok * p.Hq + head] : p.q_scale[0];
}

template <int KIND>
__device__ __forceinline__ float kscale_of(const KParams& p, const SeqCtx& s, int key, float* vsc) {
  if constexpr (KIND != KIND_F8) {
    *vsc = 1.f;
    return 1.f;
  } else {
    if ((p.scale_mode & 3) == 2) {        // per (physical page, kv head); page_size >= 64
      const int page = page_of(p, s, key);
      *vsc = p.v_scale[page * p.Hkv + s.g];
      return p.k_scale[page * p.Hkv + s.g];
    }
    *vsc = p.v_scale[0];
    return p.k_scale[0];
  }
}

// QK operands of lane group h from a row: K-step ks holds dims 32 ks + 8 h ..+7
// (bf16, fp8) or 16 (ks / 4) + 4 h + ks % 4 (fp32).  `at` points at the row's
// dim 8 h (bf16, fp8) or 4 h (fp32) already; nullptr loads zeros.
//
// PAIRED (fp8 only): K-steps 2c and 2c + 1 hold dims 64 c + 16 h ..+7 and
// ..+8 ..+15, so that a lane reads 16 contiguous bytes per pair of K-steps.
// The dot product over d does not depend on which dims meet in a K-step, so Q
// and K only have to agree: the sequence-Q-block path loads both this way
// (measured 1-2% faster for fp8 decode on MI355X); the other small paths
// (measured 2.5% slower with it) and the large path keep the plain order.
template <int KIND>
constexpr bool kPairedK = KIND == KIND_F8;
template <int KIND, bool PAIRED = false>
__device__ __forceinline__ int lane_dim_bytes(int h) {
  return KIND == KIND_F32 ? 16 * h : (KIND == KIND_BF16 || PAIRED ? 16 * h : 8 * h);
}

template <int KIND, int D, bool PAIRED = false>
__device__ __forceinline__ void load_qk_at(const char* at, typename QKOpT<KIND>::T (&op)[Cfg<KIND, D>::KSQ]) {
  using C = Cfg<KIND, D>;
  if constexpr (KIND == KIND_F8 && PAIRED) {
#pragma unroll
    for (int c = 0; c < C::KSQ / 2; ++c) {
      const u32x4 v = at ? *reinterpret_cast<const u32x4*>(at + 64 * c) : u32x4{0, 0, 0, 0};
      op[2 * c] = __builtin_bit_cast(long, u32x2{v[0], v[1]});
      op[2 * c + 1] = __builtin_bit_cast(long, u32x2{v[2], v[3]});
    }
  } else if constexpr (KIND == KIND_BF16) {
#pragma unroll
    for (int ks = 0; ks < C::KSQ; ++ks) {
      u32x4 v = at ? *reinterpret_cast<const u32x4*>(at + 64 * ks) : u32x4{0, 0, 0, 0};
      op[ks] = __builtin_bit_cast(bf16x8, v);
    }
  } else if constexpr (KIND == KIND_F8) {
#pragma unroll
    for (int ks = 0; ks < C::KSQ; ++ks) op[ks] = at ? *reinterpret_cast<const long*>(at + 32 * ks) : 0L;
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      f32x4 v = at ? *reinterpret_cast<const f32x4*>(at + 64 * c) : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) op[4 * c + i] = v[i];
    }
  }
}

template <int KIND, int D, bool PAIRED = false>
__device__ __forceinline__ void load_qk_row(const char* row, int h,
                                            typename QKOpT<KIND>::T (&op)[Cfg<KIND, D>::KSQ]) {
  load_qk_at<KIND, D, PAIRED>(row ? row + lane_dim_bytes<KIND, PAIRED>(h) : nullptr, op);
}

// ---------------------------------------------------------------------------
// masking of one S^T tile held by a lane: keys J0 + 16 mb + 4 h + j, query row
// at absolute position `pos`.
// ---------------------------------------------------------------------------
struct RowMask {
  int pos, left;    // causal bound and window start of this lane's row
  bool bit;         // block-mask bit of (row's query tile, the unit's key tile)
  float qs;         // FP8 Q scale of this lane's row (1 otherwise)
};

// The mask and scale parameters a tile loop tests on every tile.
struct TileParams {
  int causal, window, landmark, has_bm;
  float sm_log2;
  __device__ __forceinline__ static TileParams of(const KParams& p) {
    return {p.causal, p.window, p.landmark, p.bm != nullptr, p.sm_log2};
  }
  // kept in registers for a whole segment (see held())
  __device__ __forceinline__ static TileParams held_of(const KParams& p) {
    return {held(p.causal), held(p.window), held(p.landmark), held((int)(p.bm != nullptr)), held(p.sm_log2)};
  }
};

// Landmark keys (j + 1) % C == 0 inside the tile [J0, J0 + 64) as a bitmap over
// key offsets; uniform across the workgroup.
__device__ __forceinline__ uint64_t landmark_bits(const TileParams& tp, int J0) {
  uint64_t m = 0;
  if (tp.landmark > 0) {
    for (int o = tp.landmark - 1 - (J0 % tp.landmark); o < kUnitKeys; o += tp.landmark) m |= 1ull << o;
  }
  return m;
}

// The landmark flags of a lane's 16 scores (bit 4 mb + j <-> key offset
// 16 mb + 4 h + j) from a tile's 64-bit landmark bitmap.
__device__ __forceinline__ uint32_t lane_bits16(uint64_t bits64, int h) {
  const uint64_t x = bits64 >> (4 * h);
  const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  return (lo & 0xFu) | ((lo >> 12) & 0xF0u) | ((hi & 0xFu) << 8) | ((hi >> 4) & 0xF000u);
}

// Visible key offsets of one row inside a tile: lo <= o < lo + span, minus the
// landmarks flagged in l16 (the lane's 16 scores).
struct ElemMask {
  int lo;
  unsigned span;
  uint32_t l16;
  __device__ __forceinline__ void init(const TileParams& tp, const RowMask& r, int J0, int nvalid, uint64_t lmk, int h) {
    int hi = nvalid;
    if (tp.causal) hi = min(hi, r.pos - J0 + 1);
    lo = tp.window > 0 ? max(0, r.left - J0) : 0;
    span = (r.bit && hi > lo) ? (unsigned)(hi - lo) : 0u;
    l16 = lmk ? lane_bits16(lmk, h) : 0u;
  }
};

// The tile needs no causal, window, length or block-mask test for any row with
// positions in [pos_min, ...] and window starts <= left_max (landmarks aside).
__device__ __forceinline__ bool unit_is_full(const TileParams& tp, int J0, int nvalid, int pos_min, int left_max) {
  if (nvalid < kUnitKeys) return false;
  if (tp.causal && J0 + kUnitKeys - 1 > pos_min) return false;
  if (tp.window > 0 && J0 < left_max) return false;
  if (tp.has_bm) return false;
  return true;
}

// Landmark keys only (the tile is otherwise fully visible): the scores whose
// slot holds a landmark for some lane group are visited, the others skipped
// by a wave-uniform test.
__device__ __forceinline__ void mask_landmarks(f32x4 (&sc)[4], uint64_t lmk, int h) {
  uint32_t any = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) any |= lane_bits16(lmk, g);
  any = __builtin_amdgcn_readfirstlane(any);
  const uint32_t l16 = lane_bits16(lmk, h);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((any >> (4 * mb + j)) & 1u) sc[mb][j] = ((l16 >> (4 * mb + j)) & 1u) ? kNegInf : sc[mb][j];
}

// ---------------------------------------------------------------------------
// online-softmax state of NB row-blocks of one wave
// ---------------------------------------------------------------------------
template <int KIND, int D, int NB>
struct WaveState {
  f32x4 acc[NB][Cfg<KIND, D>::MD];
  // reference max m of the log2-domain scores of this lane's row, kept as
  // nmr = -m (0 while m = -inf) and thr = m + kRescaleSlack (-inf while m = -inf)
  float nmr[NB], thr[NB];
  float lsum[NB];     // this lane's share of the running sum (reduced at the end)
  f32x4 lacc[NB];     // or: the row's whole running sum, accumulated by MFMA
  __device__ __forceinline__ float m2(int nb) const { return thr[nb] == kNegInf ? kNegInf : -nmr[nb]; }
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      nmr[nb] = 0.f;
      thr[nb] = kNegInf;
      lsum[nb] = 0.f;
      lacc[nb] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int md = 0; md < Cfg<KIND, D>::MD; ++md) acc[nb][md] = f32x4{0, 0, 0, 0};
    }
  }
};

// Online softmax update of one row-block.  `s` holds raw scores Q.K (masked =
// -inf) and is overwritten by the probabilities 2^(cs * s - m); cs > 0 is the
// log2-domain score scale.  The reference max m of a row moves only when the
// row's running max exceeds it by more than kRescaleSlack, so in the common
// case the accumulator is not rescaled at all and the probabilities stay
// below 2^kRescaleSlack (exact in the result: l and O use the same m).
constexpr float kRescaleSlack = 8.f;

template <int KIND, int D, int NB, bool VSUM = true>
__device__ __forceinline__ void softmax_update(WaveState<KIND, D, NB>& st, int nb, f32x4 (&s)[4], float cs) {
  // this lane's 16 scores (the row's other 48 sit in lanes n + 16, 32, 48)
  const float m0 = max3_nonan(s[0][0], s[0][1], s[0][2]), m1 = max3_nonan(s[0][3], s[1][0], s[1][1]);
  const float m2 = max3_nonan(s[1][2], s[1][3], s[2][0]), m3 = max3_nonan(s[2][1], s[2][2], s[2][3]);
  const float m4 = max3_nonan(s[3][0], s[3][1], s[3][2]);
  const float mx = max_nonan(max3_nonan(m0, m1, m2), max3_nonan(m3, m4, s[3][3]));
  // The threshold is the same in the four lanes of a row, so some lane's max
  // exceeds it exactly when the row's max does: the cross-lane reduction is
  // needed only on that (rare) path.  cs > 0, so a row with no visible key
  // keeps its max at -inf and never grows.
  if (__ballot(mx * cs > st.thr[nb]) != 0) {            // wave-uniform, rare after the first tiles
    const float m_cand = row_max4(mx) * cs;
    const bool grow = m_cand > st.thr[nb];
    const float m_old = st.m2(nb);
    const float m_new = grow ? m_cand : m_old;
    // a row that had no visible key yet holds l = 0 and O = 0: nothing to
    // rescale (so a segment's first tile skips the multiplies altogether)
    if (__ballot(grow && m_old != kNegInf) != 0) {
      const float alpha = m_old == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_old - m_new);
      if constexpr (VSUM) st.lsum[nb] *= alpha;
      else st.lacc[nb] *= alpha;
#pragma unroll
      for (int md = 0; md < Cfg<KIND, D>::MD; ++md) st.acc[nb][md] *= alpha;
    }
    st.nmr[nb] = m_new == kNegInf ? 0.f : -m_new;
    st.thr[nb] = m_new + kRescaleSlack;
  }
  const float nmref = st.nmr[nb];
  float sum = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][j], cs, nmref));
      s[mb][j] = e;
      if constexpr (VSUM) sum = mb + j == 0 ? e : sum + e;
    }
  if constexpr (VSUM) st.lsum[nb] += sum;
}

// An all-ones bf16 A operand: MFMA against a P^T operand yields the P row sums
// (the same bf16 probabilities PV uses) replicated over the output rows.
__device__ __forceinline__ bf16x8 ones_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
}

// P^T operand (bf16) of PV K-step ks2: slot t = key 32 ks2 + 16 (t / 4) + 4 h + t % 4.
__device__ __forceinline__ bf16x8 p_operand(const f32x4 (&pr)[4], int ks2, float vsc) {
  u32x4 w;
  w[0] = pack_bf16x2(pr[2 * ks2][0] * vsc, pr[2 * ks2][1] * vsc);
  w[1] = pack_bf16x2(pr[2 * ks2][2] * vsc, pr[2 * ks2][3] * vsc);
  w[2] = pack_bf16x2(pr[2 * ks2 + 1][0] * vsc, pr[2 * ks2 + 1][1] * vsc);
  w[3] = pack_bf16x2(pr[2 * ks2 + 1][2] * vsc, pr[2 * ks2 + 1][3] * vsc);
  return __builtin_bit_cast(bf16x8, w);
}

// V^T operand for element md from the 8 V row pieces of one PV K-step
// (index half * 4 + j, each MD bf16 = MD / 2 words): slot t <- piece t, element md.
template <int MD>
__device__ __forceinline__ bf16x8 v_operand(const unsigned (&vr)[8][MD / 2], int md) {
  u32x4 w;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const unsigned a = vr[2 * u][md >> 1], b = vr[2 * u + 1][md >> 1];
    w[u] = (md & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
  }
  return __builtin_bit_cast(bf16x8, w);
}

// A raw V piece: MD consecutive elements of one V row (16 B of bf16 or 8 B of
// fp8 for d = 128), converted to bf16 words only when the PV operand is built.
template <int KIND, int MD> struct VRawT;
template <> struct VRawT<KIND_BF16, 8> { using T = u32x4; };
template <> struct VRawT<KIND_BF16, 4> { using T = u32x2; };
template <> struct VRawT<KIND_F8, 8> { using T = u32x2; };
template <> struct VRawT<KIND_F8, 4> { using T = unsigned; };

template <int KIND, int MD>
__device__ __forceinline__ typename VRawT<KIND, MD>::T load_v_raw(const char* row, int e0) {
  return *reinterpret_cast<const typename VRawT<KIND, MD>::T*>(row + e0 * (KIND == KIND_BF16 ? 2 : 1));
}

template <int KIND, int MD>
__device__ __forceinline__ void v_words(const typename VRawT<KIND, MD>::T& r, unsigned (&out)[MD / 2]) {
  if constexpr (KIND == KIND_BF16) {
#pragma unroll
    for (int i = 0; i < MD / 2; ++i) out[i] = r[i];
  } else if constexpr (MD == 8) {
    out[0] = f8x2_to_bf16x2(r[0]);
    out[1] = f8x2_to_bf16x2<true>(r[0]);
    out[2] = f8x2_to_bf16x2(r[1]);
    out[3] = f8x2_to_bf16x2<true>(r[1]);
  } else {
    out[0] = f8x2_to_bf16x2(r);
    out[1] = f8x2_to_bf16x2<true>(r);
  }
}

// ---------------------------------------------------------------------------
// final write of one lane's row: O = acc / l (out dtype) and LSE; or the
// normalised partial (fp32) and its LSE into a slot.  `o` holds the lane's
// MD x 4 values in accumulator order.
// ---------------------------------------------------------------------------
// Head dim held by accumulator element j of O^T M-block md in lane group h.
// TRV: V^T operands read by transpose loads from a row-major V tile (dims 16 md + m).
template <int KIND, int D, bool TRV = false>
__device__ __forceinline__ int out_dim(int h, int j, int md) {
  if constexpr (TRV) return 16 * md + 4 * h + j;
  else if constexpr (KIND == KIND_F32) return 4 * (4 * h + j) + (md & 3) + 64 * (md >> 2);
  else return Cfg<KIND, D>::MD * (4 * h + j) + md;
}

template <int KIND, int D, bool TRV = false>
__device__ __forceinline__ void write_row(const KParams& p, const QBlock& x, int r, int h,
                                          const f32x4 (&acc)[Cfg<KIND, D>::MD], float inv_l,
                                          float lse, bool final_out, int slot) {
  constexpr int MD = Cfg<KIND, D>::MD;
  const int tok = x.q0 + x.t0 + r / p.qbh, head = x.g * p.G + r % p.qbh;
  if constexpr (TRV) {
    if (final_out) {
      char* o = reinterpret_cast<char*>(p.out) + (tok * p.o_st + head * p.o_sh) * 2;
#pragma unroll
      for (int md = 0; md < MD; ++md)
        *reinterpret_cast<u32x2*>(o + out_dim<KIND, D, true>(h, 0, md) * 2) =
            u32x2{pack_bf16x2(acc[md][0] * inv_l, acc[md][1] * inv_l), pack_bf16x2(acc[md][2] * inv_l, acc[md][3] * inv_l)};
      if (h == 0) p.lse[tok * p.l_st + head * p.l_sh] = lse;
    } else {
      float* o = p.part_o + ((int64_t)slot * p.slot_rows + r) * D;
      if (p.fused) {
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int i = 0; i < 4; ++i) store_coherent(o + out_dim<KIND, D, true>(h, 0, md) + i, acc[md][i] * inv_l);
        if (h == 0) store_coherent(p.part_lse + slot * p.slot_rows + r, lse);
      } else {
#pragma unroll
        for (int md = 0; md < MD; ++md)
          *reinterpret_cast<f32x4*>(o + out_dim<KIND, D, true>(h, 0, md)) = acc[md] * inv_l;
        if (h == 0) p.part_lse[slot * p.slot_rows + r] = lse;
      }
    }
    return;
  }
  if (final_out) {
    if constexpr (KIND == KIND_F32) {
      float* o = reinterpret_cast<float*>(p.out) + tok * p.o_st + head * p.o_sh;
#pragma unroll
      for (int gd = 0; gd < D / 64; ++gd)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[4 * gd + i][j] * inv_l;
          *reinterpret_cast<f32x4*>(o + out_dim<KIND, D>(h, j, 4 * gd)) = v;
        }
    } else {
      char* o = reinterpret_cast<char*>(p.out) + (tok * p.o_st + head * p.o_sh) * 2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        unsigned w[MD / 2];
#pragma unroll
        for (int i = 0; i < MD / 2; ++i) w[i] = pack_bf16x2(acc[2 * i][j] * inv_l, acc[2 * i + 1][j] * inv_l);
        char* dst = o + out_dim<KIND, D>(h, j, 0) * 2;
        if constexpr (MD == 8) *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
        else *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
      }
    }
    if (h == 0) p.lse[tok * p.l_st + head * p.l_sh] = lse;
  } else {
    float* o = p.part_o + ((int64_t)slot * p.slot_rows + r) * D;
    if (p.fused) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int md = 0; md < MD; ++md) store_coherent(o + out_dim<KIND, D>(h, j, md), acc[md][j] * inv_l);
      if (h == 0) store_coherent(p.part_lse + slot * p.slot_rows + r, lse);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int md = 0; md < MD; ++md) o[out_dim<KIND, D>(h, j, md)] = acc[md][j] * inv_l;
      if (h == 0) p.part_lse[slot * p.slot_rows + r] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// active-tile list of a block-sparse Q-block (wave 0 builds, all wait):
// list[i] = tile of active unit u_start + i, for i < n.
// ---------------------------------------------------------------------------
__device__ void build_tile_list(const KParams& p, const QBlock& x, int t_lo, int t_hi, int u_start,
                                int n, short* list) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int rank0 = 0;
    for (int base = t_lo; base <= t_hi && rank0 < u_start + n; base += 64) {
      const int t = base + lane;
      const bool act = t <= t_hi && mask_union(p, x.b, x.g, x.pos_lo, x.pos_hi, t);
      const unsigned long long bal = __ballot(act);
      const int rank = rank0 + __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
      if (act && rank >= u_start && rank < u_start + n) list[rank - u_start] = (short)t;
      rank0 += __popcll(bal);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// small Q-blocks (<= 16 rows): one wave runs a contiguous run of units with
// operands loaded straight from HBM into registers.  Each wave keeps exactly
// one tile (32 KiB of K and V) in flight: issue the tile's loads, consume
// them, then issue the next tile.  Measured on MI355X with this access
// pattern, one tile in flight per wave sustains ~6.2 TB/s while also
// prefetching the next tile during compute drops to ~3.7 TB/s (the extra
// outstanding requests congest the memory system); only the next tile's page
// number is fetched ahead (a scalar load).  An fp8 tile is 16 KiB: there the
// next tile's K is issued right after this tile's QK and its V right after
// this tile's PV, which keeps at most one bf16 tile's worth outstanding.
// ---------------------------------------------------------------------------
template <int KIND, int D>
struct SmallRegs {
  using C = Cfg<KIND, D>;
  static constexpr int MD = C::MD;
  typename QKOpT<KIND>::T kA[4][C::KSQ];
  // bf16 / fp8: V row pieces per PV K-step (ks2) and piece (half * 4 + j)
  typename std::conditional<KIND == KIND_F32, int, typename VRawT<KIND == KIND_F32 ? KIND_BF16 : KIND, MD>::T>::type
      vr[KIND == KIND_F32 ? 1 : 2][KIND == KIND_F32 ? 1 : 8];
  // fp32: V rows (mb, j), dims 64 gd + 4 n
  f32x4 vf[KIND == KIND_F32 ? 4 : 1][KIND == KIND_F32 ? 4 : 1][KIND == KIND_F32 ? D / 64 : 1];
};

// QK operands from a buffer: K-step ks of lane group h at voff + (ks part), soff.
template <int KIND, int D, bool PAIRED = false, bool TEMPORAL = false>
__device__ __forceinline__ void bload_qk(const char* r, uint32_t voff, uint32_t soff,
                                         typename QKOpT<KIND>::T (&op)[Cfg<KIND, D>::KSQ]) {
  using C = Cfg<KIND, D>;
  if constexpr (KIND == KIND_F8 && PAIRED) {
#pragma unroll
    for (int c = 0; c < C::KSQ / 2; ++c) {
      const u32x4 v = gload16(r, voff + 64 * c, soff);
      op[2 * c] = __builtin_bit_cast(long, u32x2{v[0], v[1]});
      op[2 * c + 1] = __builtin_bit_cast(long, u32x2{v[2], v[3]});
    }
  } else if constexpr (KIND == KIND_BF16) {
#pragma unroll
    for (int ks = 0; ks < C::KSQ; ++ks)
      op[ks] = __builtin_bit_cast(bf16x8, TEMPORAL ? gload16t(r, voff + 64 * ks, soff) : gload16(r, voff + 64 * ks, soff));
  } else if constexpr (KIND == KIND_F8) {
#pragma unroll
    for (int ks = 0; ks < C::KSQ; ++ks) op[ks] = __builtin_bit_cast(long, gload8(r, voff + 32 * ks, soff));
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const f32x4 v = __builtin_bit_cast(f32x4, gload16(r, voff + 64 * c, soff));
#pragma unroll
      for (int i = 0; i < 4; ++i) op[4 * c + i] = v[i];
    }
  }
}

template <int KIND, int MD>
__device__ __forceinline__ typename VRawT<KIND, MD>::T bload_v(const char* r, uint32_t voff, uint32_t soff) {
  using T = typename VRawT<KIND, MD>::T;
  if constexpr (sizeof(T) == 16) return gload16(r, voff, soff);
  else if constexpr (sizeof(T) == 8) return gload8nt(r, voff, soff);
  else return gload4(r, voff, soff);
}

template <int KIND, int D, bool FAST, bool PAIRED = false, bool TEMPORAL = false>
__device__ __forceinline__ void small_load_k(const KParams& p, const SeqCtx& s, const Tile<Cfg<KIND, D>::ELT, FAST>& t,
                                             SmallRegs<KIND, D>& r, int n, int h) {
  if constexpr (FAST) {
    // The tile lies inside one page, so rows past the sequence end are still
    // cache memory: read them unclamped (their scores are masked to -inf by
    // select, never used).  Uniform row bases + one lane offset keep every
    // load in the scalar-base form.
    const uint32_t lane = (uint32_t)n * t.kss + lane_dim_bytes<KIND, PAIRED>(h);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) bload_qk<KIND, D, PAIRED, TEMPORAL>(t.kb + 16 * mb * t.kss, lane, 0u, r.kA[mb]);
  } else {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) load_qk_row<KIND, D, PAIRED>(t.krow(p, s, 16 * mb + n), h, r.kA[mb]);
  }
}

template <int KIND, int D, bool FAST>
__device__ __forceinline__ void small_load_v(const KParams& p, const SeqCtx& s, const Tile<Cfg<KIND, D>::ELT, FAST>& t,
                                             SmallRegs<KIND, D>& r, int n, int h) {
  constexpr int MD = Cfg<KIND, D>::MD;
  constexpr int ELT = Cfg<KIND, D>::ELT;
  if constexpr (KIND == KIND_F32) {
    // rows 16 mb + 4 h + j, dims 64 gd + 4 n
    if constexpr (FAST) {
      const bool full = t.nvalid == kUnitKeys;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kt = 16 * mb + 4 * h + j;
          const uint32_t voff = full ? (uint32_t)(4 * h) * t.vss + 16 * n
                                     : (uint32_t)min(kt, t.nvalid - 1) * t.vss + 16 * n;
          const uint32_t soff = full ? (uint32_t)(16 * mb + j) * t.vss : 0u;
#pragma unroll
          for (int gd = 0; gd < D / 64; ++gd)
            r.vf[mb][j][gd] = __builtin_bit_cast(f32x4, gload16(t.vb, voff + 256 * gd, soff));
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const char* row = t.vrow(p, s, 16 * mb + 4 * h + j) + 16 * n;
#pragma unroll
          for (int gd = 0; gd < D / 64; ++gd) r.vf[mb][j][gd] = *reinterpret_cast<const f32x4*>(row + 256 * gd);
        }
    }
  } else {
    // piece (ks2, pc): row 32 ks2 + 16 (pc / 4) + 4 h + pc % 4, dims MD n ..
    if constexpr (FAST) {
      // unclamped as for K; rows past the sequence end may hold anything (NaN
      // included) and would poison O through 0 * NaN, so they are zeroed
      const uint32_t lane = (uint32_t)(4 * h) * t.vss + MD * n * ELT;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int pc = 0; pc < 8; ++pc)
          r.vr[ks2][pc] = bload_v<KIND, MD>(t.vb + (32 * ks2 + 16 * (pc >> 2) + (pc & 3)) * t.vss, lane, 0u);
      if (t.nvalid < kUnitKeys) {                        // uniform: the sequence's last tile
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
          for (int pc = 0; pc < 8; ++pc)
            if (32 * ks2 + 16 * (pc >> 2) + 4 * h + (pc & 3) >= t.nvalid) r.vr[ks2][pc] = {};
      }
    } else {
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int pc = 0; pc < 8; ++pc)
          r.vr[ks2][pc] = load_v_raw<KIND, MD>(t.vrow(p, s, 32 * ks2 + 16 * (pc >> 2) + 4 * h + (pc & 3)), MD * n);
    }
  }
}

// Apply the per-element mask of one row-block (lane's row) to the scores.
__device__ __forceinline__ void mask_scores(f32x4 (&sc)[4], const ElemMask& em, int h) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = 16 * mb + 4 * h + j;
      const bool ok = ((unsigned)(o - em.lo) < em.span) && !((em.l16 >> (4 * mb + j)) & 1u);
      sc[mb][j] = ok ? sc[mb][j] : kNegInf;
    }
}
// The same mask as an additive bias (0 where visible, -inf where masked).
__device__ __forceinline__ void mask_bias(f32x4 (&bias)[4], const ElemMask& em, int h) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = 16 * mb + 4 * h + j;
      const bool ok = ((unsigned)(o - em.lo) < em.span) && !((em.l16 >> (4 * mb + j)) & 1u);
      bias[mb][j] = ok ? 0.f : kNegInf;
    }
}

// Q operands of a small Q-block, staged in LDS (element ks * 64 + lane holds
// lane's operand of K-step ks) or held in the lane's registers.
template <int KIND, int D>
struct QFromLds {
  const typename QKOpT<KIND>::T* q;
  __device__ __forceinline__ typename QKOpT<KIND>::T operator()(int ks, int lane) const { return q[ks * 64 + lane]; }
};
template <int KIND, int D>
struct QFromRegs {
  const typename QKOpT<KIND>::T* q;
  __device__ __forceinline__ typename QKOpT<KIND>::T operator()(int ks, int) const { return q[ks]; }
};

// Scores of one tile, S^T = K Q^T, masked and passed through the online
// softmax: leaves P (unnormalised probabilities) in sc; returns the tile's V scale.
// rows_mixed: the 16 rows belong to several kv heads, so the element mask
// (rm.bit = 0 for rows of other heads) runs on every tile.
template <int KIND, int D, bool FAST, class QSrc>
__device__ __forceinline__ float small_scores(const KParams& p, const SeqCtx& s, const QBlock& x,
                                              const Tile<Cfg<KIND, D>::ELT, FAST>& tc, const SmallRegs<KIND, D>& r,
                                              const QSrc& qsrc, RowMask& rm, int bm_head, int pos_min, int left_max,
                                              WaveState<KIND, D, 1>& st, int lane, f32x4 (&sc)[4],
                                              bool rows_mixed = false, KvScales ts = KvScales{1.f, 1.f, false}) {
  using C = Cfg<KIND, D>;
  const int h = lane >> 4;
  const int J0 = tc.J0;
  float vsc;
  float ksc;
  if (KIND == KIND_F8 && ts.valid) {
    ksc = ts.k;
    vsc = ts.v;
  } else if constexpr (FAST) {
    ksc = kscale_at_page<KIND>(p, s, tc.page, &vsc);
  } else {
    ksc = kscale_of<KIND>(p, s, J0, &vsc);
  }
  if (p.bm) {
    const int kt = J0 / p.bm_tile, qt = rm.pos / p.bm_tile;
    rm.bit = kt < p.bm_nk && qt < p.bm_nq &&
             p.bm[x.b * p.bm_sb + bm_head * p.bm_sh + qt * p.bm_sq + kt * p.bm_sk] != 0;
  }
  // S^T = K Q^T (Q operands re-read from LDS)
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) sc[mb] = f32x4{0, 0, 0, 0};
  if constexpr (KIND == KIND_F8 && D == 128) {
    const i32x8 qc = cat4(qsrc(0, lane), qsrc(1, lane), qsrc(2, lane), qsrc(3, lane));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) sc[mb] = mfma_qk128(cat4(r.kA[mb][0], r.kA[mb][1], r.kA[mb][2], r.kA[mb][3]), qc, sc[mb]);
  } else {
#pragma unroll
    for (int ks = 0; ks < C::KSQ; ++ks) {
      const typename QKOpT<KIND>::T qb = qsrc(ks, lane);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) sc[mb] = mfma_qk(r.kA[mb][ks], qb, sc[mb]);
    }
  }
  const TileParams tp = TileParams::of(p);
  const uint64_t lmk = landmark_bits(tp, J0);
  const bool full = !rows_mixed && unit_is_full(tp, J0, tc.nvalid, pos_min, left_max);
  float cs = tp.sm_log2;
  if constexpr (KIND == KIND_F8) cs *= rm.qs * ksc;
  if (!full) {
    ElemMask em;
    em.init(tp, rm, J0, tc.nvalid, lmk, h);
    mask_scores(sc, em, h);
  } else if (lmk) {
    mask_landmarks(sc, lmk, h);
  }
  softmax_update<KIND, D, 1>(st, 0, sc, cs);
  return vsc;
}

// O^T += V^T P^T for one tile
template <int KIND, int D>
__device__ __forceinline__ void small_pv(const SmallRegs<KIND, D>& r, const f32x4 (&sc)[4], float vsc,
                                         WaveState<KIND, D, 1>& st) {
  constexpr int MD = Cfg<KIND, D>::MD;
  if constexpr (KIND == KIND_F32) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int md = 0; md < MD; ++md)
          st.acc[0][md] = __builtin_amdgcn_mfma_f32_16x16x4f32(r.vf[mb][j][md >> 2][md & 3], sc[mb][j],
                                                                st.acc[0][md], 0, 0, 0);
  } else {
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      unsigned w[8][MD / 2];
#pragma unroll
      for (int pc = 0; pc < 8; ++pc) v_words<KIND, MD>(r.vr[ks2][pc], w[pc]);
      const bf16x8 pb = p_operand(sc, ks2, vsc);
#pragma unroll
      for (int md = 0; md < MD; ++md) st.acc[0][md] = mfma_pv(v_operand<MD>(w, md), pb, st.acc[0][md]);
    }
  }
}

template <int KIND, int D, bool FAST, class QSrc>
__device__ __forceinline__ void small_compute(const KParams& p, const SeqCtx& s, const QBlock& x,
                                              const Tile<Cfg<KIND, D>::ELT, FAST>& tc, const SmallRegs<KIND, D>& r,
                                              const QSrc& qsrc, RowMask& rm, int bm_head,
                                              int pos_min, int left_max, WaveState<KIND, D, 1>& st, int lane) {
  f32x4 sc[4];
  const float vsc = small_scores<KIND, D, FAST>(p, s, x, tc, r, qsrc, rm, bm_head, pos_min, left_max, st, lane, sc);
  small_pv<KIND, D>(r, sc, vsc, st);
}

// ---------------------------------------------------------------------------
// fused combine ("Triton-TLE rewrite of Tencent HPC-Ops Attention", §3.3: each
// split publishes its partial state and a completion counter tells the last
// one to merge; the AMD counterpart of the page's cluster merge is a
// device-scope counter per Q-block).  Called by the whole workgroup after it
// wrote its partial of split Q-block q (device-coherent stores, complete
// before the counter moves); the workgroup that brings the counter to ns
// merges all ns partials (device-coherent loads) and writes the output rows.
// No workgroup waits on another.
// ---------------------------------------------------------------------------
template <int KIND, int D>
__device__ void finish_split(const KParams& p, int q, const QBlock& x, int ns, int sb) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // the flag sits in the dynamic block past the merge's 256 reduction slots
  // (a static variable would take LDS that the lean build's stages fill)
  int& last = *reinterpret_cast<int*>(smem + 256 * sizeof(MergeState));
  // Publication: every thread's partial stores (device-coherent) are complete
  // before the barrier, and after it one thread counts the piece with an
  // agent-scope release; the workgroup that brings the count to ns acquires
  // at agent scope before it reads the other pieces.  (Release and acquire
  // order the counter against the pieces in the memory model; the waits make
  // the other waves' stores part of what the release publishes.)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(p.done + q, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == ns - 1;
  __syncthreads();
  if (last) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    merge_qblock<D, KIND == KIND_F32, true>(p, x, ns, sb, reinterpret_cast<MergeState*>(smem));
  }
  __syncthreads();
}

// One tile in flight per wave: the second wave on each SIMD (two workgroups
// per compute unit) computes while this one waits for its loads.
template <int KIND, int D, bool FAST>
__device__ __forceinline__ void small_run(const KParams& p, const SeqCtx& s, const QBlock& x, const short* list,
                                          int c0, int t_lo, int a, int b,
                                          const typename QKOpT<KIND>::T* qlds, RowMask rm,
                                          int bm_head, int pos_min, int left_max, WaveState<KIND, D, 1>& st,
                                          int lane) {
  using C = Cfg<KIND, D>;
  const int n = lane & 15, h = lane >> 4;
  for (int u = a; u < b; ++u) {
    // wave-uniform: keeps tile addressing in scalar registers
    const int tile = __builtin_amdgcn_readfirstlane(p.bm ? (int)list[u - c0] : t_lo + u);
    Tile<C::ELT, FAST> t;
    SmallRegs<KIND, D> r;
    t.init(p, s, tile);
    small_load_k<KIND, D, FAST, false, true>(p, s, t, r, n, h);   // bf16 K temporal (see gload16t)
    small_load_v<KIND, D, FAST>(p, s, t, r, n, h);
    small_compute<KIND, D, FAST>(p, s, x, t, r, QFromLds<KIND, D>{qlds}, rm, bm_head, pos_min, left_max, st, lane);
  }
}

template <int KIND, int D, bool FAST>
__device__ PA_SEGMENT_FN void small_segment(uint64_t pk, const QBlock x, int t_lo, int t_hi, int u0,
                                                       int u1, bool final_out, int slot) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const KParams& p = kparams_at(pk);
  using C = Cfg<KIND, D>;
  constexpr int MD = C::MD;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, h = lane >> 4;
  short* list = reinterpret_cast<short*>(smem + Lds<KIND, D, FAST>::DYN - kMaskListCap * 2);

  SeqCtx s{x.b, x.g, x.ctx, t_lo, p.bt + (int64_t)x.b * p.bt_stride};
  // this lane's query row
  const bool row_ok = n < x.rows;
  const int r = row_ok ? n : 0;
  const int tok = x.q0 + x.t0 + r / p.G, head = x.g * p.G + r % p.G;
  // Q operands of the 16 rows, in operand order [ks][lane], after the merge area
  using QT = typename QKOpT<KIND>::T;
  QT* qlds = reinterpret_cast<QT*>(smem + C::QOFF);
  if (wave == 0) {
    QT qB[C::KSQ];
    load_qk_row<KIND, D>(row_ok ? reinterpret_cast<const char*>(p.q) + (tok * p.q_st + head * p.q_sh) * C::ELT
                                : nullptr, h, qB);
#pragma unroll
    for (int ks = 0; ks < C::KSQ; ++ks) qlds[ks * 64 + lane] = qB[ks];
  }
  __syncthreads();
  RowMask rm;
  rm.pos = x.ctx - x.ql + x.t0 + r / p.G;
  rm.left = p.window > 0 ? window_left(p, rm.pos) : 0;
  rm.bit = true;
  rm.qs = qscale_of<KIND>(p, tok, head);
  const int pos_min = x.pos_lo;
  const int left_max = p.window > 0 ? window_left(p, x.pos_hi) : 0;
  const int bm_head = p.bm && p.bm_heads != 1 ? head : 0;

  WaveState<KIND, D, 1> st;
  st.init();
  // units are taken in chunks of at most kMaskListCap (the list capacity);
  // inside a chunk the waves take contiguous quarter runs
  for (int c0 = u0; c0 < u1; c0 += kMaskListCap) {
    const int cn = min(kMaskListCap, u1 - c0);
    if (p.bm) build_tile_list(p, x, t_lo, t_hi, c0, cn, list);
    const int a = c0 + (cn * wave) / kWaves, b = c0 + (cn * (wave + 1)) / kWaves;
    if (a < b) small_run<KIND, D, FAST>(p, s, x, list, c0, t_lo, a, b, qlds, rm, bm_head, pos_min, left_max, st, lane);
    if (p.bm) __syncthreads();                 // list reuse
  }

  // merge the four waves' states through LDS: m, l per row; acc per row x dims
  float l = st.lsum[0];
  l = row_sum4(l);
  float* mrg = reinterpret_cast<float*>(smem);
  float* ms = mrg;                                     // [wave][16]
  float* ls = mrg + kWaves * 16;                       // [wave][16]
  float* os = mrg + 2 * kWaves * 16;                   // [wave][16][D]
  if (h == 0) {
    ms[wave * 16 + n] = st.m2(0);
    ls[wave * 16 + n] = l;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int md = 0; md < MD; ++md) os[(wave * 16 + n) * D + out_dim<KIND, D>(h, j, md)] = st.acc[0][md][j];
  __syncthreads();
  // thread -> (row, 8 dims)
  constexpr int TPR = D / 8;                           // threads per row
  for (int idx = threadIdx.x; idx < 16 * TPR; idx += kThreads) {
    const int row = idx / TPR, d0 = (idx % TPR) * 8;
    if (row >= x.rows) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ms[w * 16 + row]);
    float L = 0.f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float c = __builtin_amdgcn_exp2f(ms[w * 16 + row] - M);
        L += ls[w * 16 + row] * c;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] += os[(w * 16 + row) * D + d0 + i] * c;
      }
    }
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    const float lse = empty ? kNegInf : (M + log2f(L)) * kLn2;
    const int tk = x.q0 + x.t0 + row / p.G, hd = x.g * p.G + row % p.G;
    if (final_out) {
      if constexpr (KIND == KIND_F32) {
        float* dst = reinterpret_cast<float*>(p.out) + tk * p.o_st + hd * p.o_sh + d0;
        *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
      } else {
        char* dst = reinterpret_cast<char*>(p.out) + (tk * p.o_st + hd * p.o_sh + d0) * 2;
        *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                                               pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
      }
      if (d0 == 0) p.lse[tk * p.l_st + hd * p.l_sh] = lse;
    } else {
      float* dst = p.part_o + ((int64_t)slot * p.slot_rows + row) * D + d0;
      if (p.fused) {
        for (int i = 0; i < 8; ++i) store_coherent(dst + i, o[i] * inv);
        if (d0 == 0) store_coherent(p.part_lse + slot * p.slot_rows + row, lse);
      } else {
        *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
        if (d0 == 0) p.part_lse[slot * p.slot_rows + row] = lse;
      }
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// A run of consecutive small Q-blocks inside one worker's range (no block
// mask).  The run's units are cut into four contiguous quarters, one per
// wave; each wave streams its tiles without pause across Q-block boundaries
// (the double-buffered loads of the next tile — K, V and its Q-block's Q
// rows — overlap the current tile's math).  A Q-block lying wholly inside a
// wave's quarter is written out directly; only the first and last Q-block of
// a quarter can be cut, and those pieces are merged once, through LDS, when
// the run ends.  Per-segment splitting would instead drain every wave's
// pipeline and synchronise the workgroup at each of the many short decode
// Q-blocks of a ragged batch.
// ---------------------------------------------------------------------------
// decode streaming with loads half a tile ahead: fp8 only.  A bf16 tile is
// twice the registers, and holding the next K through the PV spills
// (measured slower); for fp8 it is ~4% faster.  (Two whole fp8 tiles in
// registers spill as well.)
template <int KIND>
constexpr bool kHalfStep = KIND == KIND_F8;

template <int KIND, int D, bool FAST>
struct StreamRec {
  int q, t_lo;
  QBlock x;
  Tile<Cfg<KIND, D>::ELT, FAST> t;
  SmallRegs<KIND, D> r;
  typename QKOpT<KIND>::T qB[Cfg<KIND, D>::KSQ];   // Q operands of the record's Q-block
};

// Where the stream stands: the Q-block of the current unit, its unit range
// [S, E), and a window of 64 page-table entries of its sequence held one per
// lane, so that a tile's page costs a register read instead of a dependent
// scalar memory load.
struct StreamCursor {
  int q, S, E, t_lo;
  QBlock x;
  int pbase;     // page-table index held by lane 0 of vpage
  int vpage;
  int nE;        // unit_prefix[q + 2], loaded ahead of the next Q-block change
};

template <int KIND, int D, bool FAST>
struct StashLayout {   // 8 pieces (2 per wave): m[16], l[16], acc[16][D] (raw), tag
  static constexpr int PIECES = 2 * kWaves;
  static constexpr bool SPLIT = Lds<KIND, D, FAST>::SPLIT_V;
  static constexpr int M = 0, Lf = PIECES * 16, ACC = 2 * PIECES * 16;
  static constexpr int FLOATS = ACC + Lds<KIND, D, FAST>::STASH_PIECES_DYN * 16 * D;
  // raw accumulator of piece k: in the dynamic block, or (split) pieces
  // kWaves.. two to a V stage
  __device__ __forceinline__ static float* acc(float* stash, int k) {
    if constexpr (SPLIT) {
      if (k >= kWaves) return reinterpret_cast<float*>(vstage<true>((k - kWaves) >> 1)) + ((k - kWaves) & 1) * 16 * D;
    }
    return stash + ACC + k * 16 * D;
  }
};

// The Q-block holding unit a: the last q in [lo, hi] with unit_prefix[q] <= a
// (unit_prefix[lo] <= a).  A 64-way search: each round probes 64 evenly
// spaced entries with one vector load, so ceil(log64(n)) dependent loads
// instead of a binary search's log2(n), which at kernel start (every worker
// searching at once, nothing else in flight) is pure latency.
__device__ __forceinline__ int find_qblock(const KParams& p, int lo, int hi, int a, int lane) {
  lo = wave_uniform(lo);
  hi = wave_uniform(hi);
  while (lo < hi) {
    const int step = (hi - lo + 64) >> 6;
    const int idx = lo + lane * step;
    const bool ok = idx <= hi && p.unit_prefix[min(idx, hi)] <= a;
    const uint64_t m = __ballot(ok);                    // lane 0 is always set
    lo = wave_uniform(lo + (63 - __builtin_clzll(m)) * step);
    hi = wave_uniform(min(hi, lo + step - 1));
  }
  return lo;
}

template <int KIND, int D, bool FAST, bool WITH_V = true>
__device__ __forceinline__ void stream_prepare(const KParams& p, StreamCursor& c, StreamRec<KIND, D, FAST>& rec,
                                               int u, int n, int h, int lane) {
  using C = Cfg<KIND, D>;
  if (u >= c.E) {                                        // next Q-block (rare: scalar loads)
    const int b_prev = c.E < 0 ? -1 : c.x.b;
    int q;
    if (c.E < 0) {                                       // first unit of the range
      q = c.q;
      while (p.unit_prefix[q + 1] <= u) ++q;
      q = wave_uniform(q);
      c.x = load_qblock(p, q);
      c.S = wave_uniform(p.unit_prefix[q]);
      c.E = wave_uniform(p.unit_prefix[q + 1]);
    } else {
      // the end of q + 1 was loaded ahead; Q-blocks without units are skipped
      q = c.q + 1;
      int S = c.E, E = c.nE;
      while (E <= u) {
        ++q;
        S = E;
        E = p.unit_prefix[q + 1];
      }
      // small Q-blocks of one sequence are its kv heads in order: the next
      // one differs only in g, otherwise its descriptor is loaded
      if (q == c.q + 1 && c.x.g + 1 < p.Hkv) c.x.g += 1;
      else c.x = load_qblock(p, wave_uniform(q));
      c.S = wave_uniform(S);
      c.E = wave_uniform(E);
    }
    c.q = wave_uniform(q);
    c.nE = c.q + 2 <= p.hdr[H_NQB] ? p.unit_prefix[c.q + 2] : 0x7fffffff;
    int t_hi;
    qblock_tiles(p, c.x.ctx, c.x.pos_lo, c.x.pos_hi, c.t_lo, t_hi);
    if (c.x.b != b_prev) c.pbase = -(1 << 30);           // the page window stays with its sequence
  }
  const QBlock& x = c.x;
  SeqCtx s{x.b, x.g, x.ctx, c.t_lo, p.bt + (int64_t)x.b * p.bt_stride};
  if (rec.q != c.q) {                                    // a new Q-block: its Q rows
    // rows past the Q-block re-read row 0: finite scores that are never written
    const int r = n < x.rows ? n : 0;
    const int tok = x.q0 + x.t0 + r / p.G, head = x.g * p.G + r % p.G;
    const char* at = reinterpret_cast<const char*>(p.q) + (tok * p.q_st + head * p.q_sh) * C::ELT;
    __builtin_assume(at != nullptr);
    load_qk_row<KIND, D>(at, h, rec.qB);
    rec.q = c.q;
    rec.x = x;
    rec.t_lo = c.t_lo;
  }
  const int tile = c.t_lo + (u - c.S);
  if constexpr (FAST) {
    const int idx = (tile * kUnitKeys) >> p.page_shift;
    if ((unsigned)(idx - c.pbase) >= 64u) {              // refill the page window
      c.pbase = idx;
      int v = s.bt_row[min(idx + lane, p.max_pages - 1)];
      // complete the load here, where it is rare: a later read of the window
      // would otherwise wait for every load in flight, tiles included
      asm volatile("" : "+v"(v));
      c.vpage = v;
    }
    int page = idx < p.max_pages ? __builtin_amdgcn_readlane(c.vpage, idx - c.pbase) : -1;
    if ((unsigned)page >= (unsigned)p.num_pages) {
      p.hdr[H_ERROR] = E_PAGE;
      page = 0;
    }
    rec.t.init_at_page(p, s, tile, page);
  } else {
    rec.t.init(p, s, tile);
  }
  // the lane's row and column come from an opaque copy of the thread id: the
  // per-lane load offsets are then rebuilt for each tile (a few VALU ops)
  // instead of being hoisted out of the loop, where under the kernel's
  // register pressure they were spilled, and the reload from scratch
  // (counted with the vector loads) made the V loads wait for the K loads
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  // bf16 K rows through the caches here (temporal, see gload16t)
  small_load_k<KIND, D, FAST, false, true>(p, s, rec.t, rec.r, tid & 15, (tid >> 4) & 3);
  if constexpr (!WITH_V) return;
  small_load_v<KIND, D, FAST>(p, s, rec.t, rec.r, tid & 15, (tid >> 4) & 3);
}

// The V rows of the record's tile.
template <int KIND, int D, bool FAST>
__device__ __forceinline__ void stream_load_v(const KParams& p, StreamRec<KIND, D, FAST>& rec, int n, int h) {
  SeqCtx s{rec.x.b, rec.x.g, rec.x.ctx, rec.t_lo, p.bt + (int64_t)rec.x.b * p.bt_stride};
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  small_load_v<KIND, D, FAST>(p, s, rec.t, rec.r, tid & 15, (tid >> 4) & 3);
}

template <int KIND, int D, bool FAST>
__device__ PA_SEGMENT_FN void small_range(uint64_t pk, int vw, const WorkerMap wm, int a, int b) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const KParams& p = kparams_at(pk);
  using C = Cfg<KIND, D>;
  using SL = StashLayout<KIND, D, FAST>;
  constexpr int MD = C::MD;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, h = lane >> 4;
  float* stash = reinterpret_cast<float*>(smem);
  int* tags = reinterpret_cast<int*>(smem + SL::FLOATS * 4);
  if (lane < 2) tags[2 * wave + lane] = -1;
  const int cnt = b - a;
  const int wa = wave_uniform(a + (cnt * wave) / kWaves), wb = wave_uniform(a + (cnt * (wave + 1)) / kWaves);

  if (wa < wb) {
    const KvScales ts = kv_scales_hoisted<KIND>(p);
    // the current piece: its Q-block, state and row mask
    int cur_q = -1;
    QBlock cx;
    RowMask rm;
    int pos_min = 0, left_max = 0;
    WaveState<KIND, D, 1> st;
    st.init();
    auto finish = [&]() {
      float l = st.lsum[0];
      l = row_sum4(l);
      const int S = p.unit_prefix[cur_q], E = p.unit_prefix[cur_q + 1];
      if (S >= wa && E <= wb) {                          // whole Q-block in this quarter: final output
        if (n < cx.rows) {
          const bool empty = !(l > 0.f);
          write_row<KIND, D>(p, cx, n, h, st.acc[0], empty ? 0.f : 1.f / l,
                             empty ? kNegInf : (st.m2(0) + log2f(l)) * kLn2, true, 0);
        }
      } else {                                           // cut piece: stash raw state for the merge
        const int k = 2 * wave + (S < wa ? 0 : 1);
        if (lane == 0) tags[k] = cur_q;
        if (h == 0) {
          stash[SL::M + k * 16 + n] = st.m2(0);
          stash[SL::Lf + k * 16 + n] = l;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int md = 0; md < MD; ++md) SL::acc(stash, k)[n * D + out_dim<KIND, D>(h, j, md)] = st.acc[0][md][j];
      }
    };
    auto scores = [&](const StreamRec<KIND, D, FAST>& rec, f32x4 (&sc)[4]) -> float {
      if (rec.q != cur_q) {
        if (cur_q >= 0) finish();
        cur_q = rec.q;
        cx = rec.x;
        st.init();
        const int r = n < cx.rows ? n : 0;
        rm.pos = cx.ctx - cx.ql + cx.t0 + r / p.G;
        rm.left = p.window > 0 ? window_left(p, rm.pos) : 0;
        rm.bit = true;
        rm.qs = qscale_of<KIND>(p, cx.q0 + cx.t0 + r / p.G, cx.g * p.G + r % p.G);
        pos_min = cx.pos_lo;
        left_max = p.window > 0 ? window_left(p, cx.pos_hi) : 0;
      }
      SeqCtx s{cx.b, cx.g, cx.ctx, rec.t_lo, p.bt + (int64_t)cx.b * p.bt_stride};
      return small_scores<KIND, D, FAST>(p, s, cx, rec.t, rec.r, QFromRegs<KIND, D>{rec.qB}, rm, 0, pos_min,
                                         left_max, st, lane, sc, false, ts);
    };
    // the Q-block of the first unit
    StreamCursor c;
    c.q = find_qblock(p, 0, p.hdr[H_NQB] - 1, wa, lane);
    c.E = -1;                                            // forces the Q-block load on the first unit
    StreamRec<KIND, D, FAST> rec;
    rec.q = -1;
    if constexpr (kHalfStep<KIND>) {
      // half a tile ahead: the next tile's K is loaded while this tile's
      // softmax and PV run, and its V while the next QK runs, so a wave
      // keeps loads in flight through its compute without holding a second
      // tile in registers
      stream_prepare<KIND, D, FAST, false>(p, c, rec, wa, n, h, lane);
      stream_load_v<KIND, D, FAST>(p, rec, n, h);
      for (int u = wa; u < wb; ++u) {
        f32x4 sc[4];
        const float vsc = scores(rec, sc);
        if (u + 1 < wb) stream_prepare<KIND, D, FAST, false>(p, c, rec, u + 1, n, h, lane);
        small_pv<KIND, D>(rec.r, sc, vsc, st);
        if (u + 1 < wb) stream_load_v<KIND, D, FAST>(p, rec, n, h);
      }
    } else {
      // one tile in flight per wave; the second wave on each SIMD (two
      // workgroups per compute unit) computes while this one waits
      for (int u = wa; u < wb; ++u) {
        stream_prepare<KIND, D, FAST>(p, c, rec, u, n, h, lane);
        f32x4 sc[4];
        const float vsc = scores(rec, sc);
        small_pv<KIND, D>(rec.r, sc, vsc, st);
      }
    }
    finish();
  }
  __syncthreads();

  // merge the cut pieces, one Q-block at a time (at most 8 pieces)
  constexpr int TPR = D / 8;
  for (int k = 0; k < SL::PIECES; ++k) {
    const int q = tags[k];
    if (q < 0) continue;
    bool first = true;
    for (int j = 0; j < k; ++j) first = first && tags[j] != q;
    if (!first) continue;
    const QBlock x = load_qblock(p, q);
    const bool final_out = p.n_splits[q] == 1;
    const int slot = final_out ? 0 : p.slot_base[q] + (vw - wm.worker_of(p.unit_prefix[q]));
    for (int idx = threadIdx.x; idx < x.rows * TPR; idx += kThreads) {
      const int row = idx / TPR, d0 = (idx % TPR) * 8;
      float M = kNegInf;
      for (int j = k; j < SL::PIECES; ++j)
        if (tags[j] == q) M = fmaxf(M, stash[SL::M + j * 16 + row]);
      float Ls = 0.f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (M != kNegInf) {
        for (int j = k; j < SL::PIECES; ++j) {
          if (tags[j] != q) continue;
          const float c = __builtin_amdgcn_exp2f(stash[SL::M + j * 16 + row] - M);
          Ls += stash[SL::Lf + j * 16 + row] * c;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] += SL::acc(stash, j)[row * D + d0 + i] * c;
        }
      }
      const bool empty = !(Ls > 0.f);
      const float inv = empty ? 0.f : 1.f / Ls;
      const float lse = empty ? kNegInf : (M + log2f(Ls)) * kLn2;
      const int tk = x.q0 + x.t0 + row / p.G, hd = x.g * p.G + row % p.G;
      if (final_out) {
        if constexpr (KIND == KIND_F32) {
          float* dst = reinterpret_cast<float*>(p.out) + tk * p.o_st + hd * p.o_sh + d0;
          *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
        } else {
          char* dst = reinterpret_cast<char*>(p.out) + (tk * p.o_st + hd * p.o_sh + d0) * 2;
          *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                                                 pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
        }
        if (d0 == 0) p.lse[tk * p.l_st + hd * p.l_sh] = lse;
      } else {
        float* dst = p.part_o + ((int64_t)slot * p.slot_rows + row) * D + d0;
        if (p.fused) {
          for (int i = 0; i < 8; ++i) store_coherent(dst + i, o[i] * inv);
          if (d0 == 0) store_coherent(p.part_lse + slot * p.slot_rows + row, lse);
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
          if (d0 == 0) p.part_lse[slot * p.slot_rows + row] = lse;
        }
      }
    }
  }
  __syncthreads();
  if (p.fused) {
    // the Q-block of each partial written above (tags lie past the merge scratch,
    // but are read before any merge anyway)
    int pend[SL::PIECES];
#pragma unroll
    for (int k = 0; k < SL::PIECES; ++k) {
      const int q = tags[k];
      bool first = q >= 0;
      for (int j = 0; j < k; ++j) first = first && tags[j] != q;
      pend[k] = first && p.n_splits[q] != 1 ? q : -1;
    }
#pragma unroll
    for (int k = 0; k < SL::PIECES; ++k)
      if (pend[k] >= 0) finish_split<KIND, D>(p, pend[k], load_qblock(p, pend[k]), p.n_splits[pend[k]],
                                               p.slot_base[pend[k]]);
  }
}

// ---------------------------------------------------------------------------
// Decode with sequence Q-blocks: one Q-block holds every query head of a
// sequence and its units are the (tile, kv head) pairs, kv head fastest.
// Wave w owns kv heads [w hpw, (w + 1) hpw), hpw = Hkv / 4, and their query
// rows: lane n of its 16-row block is token n / (hpw G), query head
// w hpw G + n % (hpw G).  The four waves walk the same tiles, each loading its
// own heads' rows of them, so the kv heads of a key row (adjacent in an NHD
// page) are read together: measured on MI355X with the decode load pattern
// alone, 6.4 TB/s against 5.5 TB/s when each wave streams one head.  Rows of
// another kv head are masked on every tile; each wave writes its own rows
// (the output, or its rows of the worker's partial slot), so no wave merges
// with another.
// ---------------------------------------------------------------------------

template <int KIND, int D, bool FAST>
__device__ PA_SEGMENT_FN void heads_range(uint64_t pk, int vw, const WorkerMap wm, int a, int b) {
  const KParams& p = kparams_at(pk);
  using C = Cfg<KIND, D>;
  const int lane = threadIdx.x & 63, wave = wave_uniform(threadIdx.x >> 6);
  const int n = lane & 15, h = lane >> 4;
  const int Hkv = wave_uniform(p.Hkv), hpw = Hkv >> 2, wr = hpw * p.G;
  const bool mixed = hpw > 1;
  const int n_qb = p.hdr[H_NQB];
  const KvScales ts = kv_scales_hoisted<KIND>(p);
  int pbase = -(1 << 30), vpage = 0, cur_b = -1;
  for (int q = find_qblock(p, 0, n_qb - 1, a, lane); q < n_qb; ++q) {
    const int S = wave_uniform(p.unit_prefix[q]), E = wave_uniform(p.unit_prefix[q + 1]);
    if (S >= b) break;
    if (E <= a || E == S) continue;                  // no units here (Combine writes an empty Q-block)
    const QBlock x = load_qblock(p, q);
    const int lo = max(a, S) - S, hi = min(b, E) - S;   // the worker's units of q, relative to S
    // this lane's row
    const int ti = n / wr, jr = n - ti * wr;
    const bool row_ok = ti < x.nt;
    const int tok = x.q0 + (row_ok ? ti : 0), head = wave * wr + jr;
    const int rkv = head / p.G;
    typename QKOpT<KIND>::T qB[C::KSQ];
    load_qk_row<KIND, D, kPairedK<KIND>>(row_ok ? reinterpret_cast<const char*>(p.q) + (tok * p.q_st + head * p.q_sh) * C::ELT
                                               : nullptr, h, qB);
    RowMask rm;
    rm.pos = x.ctx - x.ql + (row_ok ? ti : 0);
    rm.left = p.window > 0 ? window_left(p, rm.pos) : 0;
    rm.qs = qscale_of<KIND>(p, tok, head);
    int t_lo = 0, t_hi = 0;
    qblock_tiles(p, x.ctx, x.pos_lo, x.pos_hi, t_lo, t_hi);
    const int pos_min = x.pos_lo, left_max = p.window > 0 ? window_left(p, x.pos_hi) : 0;
    SeqCtx s{x.b, 0, x.ctx, t_lo, p.bt + (int64_t)x.b * p.bt_stride};
    if (x.b != cur_b) {
      pbase = -(1 << 30);
      cur_b = x.b;
    }
    WaveState<KIND, D, 1> st;
    st.init();
    // the page of a tile, from a window of 64 page-table entries held one per
    // lane (a register read, not a dependent load, for most tiles)
    auto page_at = [&](int tile) {
      int page = 0;
      if constexpr (FAST) {
        const int idx = (tile * kUnitKeys) >> p.page_shift;
        if ((unsigned)(idx - pbase) >= 64u) {            // refill the window (rare)
          pbase = idx;
          int v = s.bt_row[min(idx + lane, p.max_pages - 1)];
          asm volatile("" : "+v"(v));
          vpage = v;
        }
        page = idx < p.max_pages ? __builtin_amdgcn_readlane(vpage, idx - pbase) : -1;
        if ((unsigned)page >= (unsigned)p.num_pages) {
          p.hdr[H_ERROR] = E_PAGE;
          page = 0;
        }
      }
      return page;
    };
    // the wave's units of q in order: (k0 = tile * Hkv, j) is kv head
    // w hpw + j of that tile, a unit of this worker when it lies in [lo, hi)
    auto valid = [&](int kk0, int j) {
      const int k = kk0 + wave * hpw + j;
      return k >= lo && k < hi;
    };
    auto advance = [&](int& kk0, int& j) {
      do {
        if (++j == hpw) {
          j = 0;
          kk0 += Hkv;
        }
      } while (kk0 < hi && !valid(kk0, j));
    };
    auto prepare = [&](Tile<C::ELT, FAST>& t, SeqCtx& sx, int kk0, int j) {
      const int tile = t_lo + kk0 / Hkv;
      sx.g = wave * hpw + j;
      if constexpr (FAST) t.init_at_page(p, sx, tile, page_at(tile));
      else t.init(p, sx, tile);
    };
    int k0 = (lo / Hkv) * Hkv, jj = 0;
    if (!valid(k0, jj)) advance(k0, jj);
    Tile<C::ELT, FAST> tc, tn;
    SeqCtx sc_ = s, sn = s;
    SmallRegs<KIND, D> r;
    // lane offsets from an opaque copy of the thread id (rebuilt per tile, not spilled)
    auto lane_n = [&]() { int tid = threadIdx.x; asm volatile("" : "+v"(tid)); return tid; };
    // fp8: the next unit's K goes out once this unit's QK has read K, and its
    // V once this unit's PV has read V.  bf16: both go out after the PV (a
    // bf16 tile is twice the bytes; issuing its K after the QK measured 1-1.5%
    // slower on MI355X at q_len 1 and 2, the fp8 schedule 1% faster than
    // issuing K late).  Either way the next QK waits for both: the compiler's
    // wait analysis also follows paths of this control flow that never run
    // (the loop entered without the first tile's loads, K loaded and V not)
    // and so waits for nearly every load in flight there.  Only K is needed,
    // but the exact wait (V left in flight through the QK and the softmax, one
    // more tile's loads outstanding per wave; built with a loop that no such
    // path reaches) measured 2-4% slower for bf16 and fp8 decode, and an
    // explicit full wait ahead of the tile's scale loads 1.5% slower for fp8:
    // the memory system does better with fewer requests in flight here, and
    // the second wave on each SIMD covers the wait.
    constexpr bool k_early = KIND == KIND_F8;
    if (k0 < hi) {
      prepare(tc, sc_, k0, jj);
      const int tid = lane_n();
      small_load_k<KIND, D, FAST, kPairedK<KIND>>(p, sc_, tc, r, tid & 15, (tid >> 4) & 3);
      small_load_v<KIND, D, FAST>(p, sc_, tc, r, tid & 15, (tid >> 4) & 3);
    }
    while (k0 < hi) {
      int nk0 = k0, nj = jj;
      advance(nk0, nj);
      const bool more = nk0 < hi;
      rm.bit = row_ok && rkv == sc_.g;                   // only this kv head's rows see the tile
      f32x4 sc[4];
      const float vsc = small_scores<KIND, D, FAST>(p, sc_, x, tc, r, QFromRegs<KIND, D>{qB}, rm, 0, pos_min,
                                                     left_max, st, lane, sc, mixed, ts);
      if (k_early && more) {
        prepare(tn, sn, nk0, nj);
        const int tid = lane_n();
        small_load_k<KIND, D, FAST, kPairedK<KIND>>(p, sn, tn, r, tid & 15, (tid >> 4) & 3);
      }
      small_pv<KIND, D>(r, sc, vsc, st);
      if (more) {
        const int tid = lane_n();
        if constexpr (!k_early) {
          prepare(tn, sn, nk0, nj);
          small_load_k<KIND, D, FAST, kPairedK<KIND>>(p, sn, tn, r, tid & 15, (tid >> 4) & 3);
        }
        small_load_v<KIND, D, FAST>(p, sn, tn, r, tid & 15, (tid >> 4) & 3);
      }
      tc = tn;
      sc_ = sn;
      k0 = nk0;
      jj = nj;
    }
    const float l = row_sum4(st.lsum[0]);
    const bool final_out = p.n_splits[q] == 1;
    const int slot = final_out ? 0 : p.slot_base[q] + (vw - wm.worker_of(S));
    if (row_ok) {
      const bool empty = !(l > 0.f);
      write_row<KIND, D>(p, x, ti * p.Hq + head, h, st.acc[0], empty ? 0.f : 1.f / l,
                         empty ? kNegInf : (st.m2(0) + log2f(l)) * kLn2, final_out, slot);
    }
    if (!final_out && p.fused) finish_split<KIND, D>(p, q, x, p.n_splits[q], p.slot_base[q]);
  }
}

// ---------------------------------------------------------------------------
// large Q-blocks (up to 128 rows): K/V tiles staged by the whole workgroup
// into LDS in MFMA-operand order, double-buffered; wave w owns rows 32 w ..
// ---------------------------------------------------------------------------
template <int KIND, int D, bool FAST>
struct Stage {
  using C = Cfg<KIND, D>;
  static constexpr int MD = C::MD;
  // per thread staging registers
  static constexpr int KCH = KIND == KIND_F32 ? (4 * (D / 16) * 64) / kThreads : (4 * C::KSQ * 64) / kThreads;
  static constexpr int VCH = KIND == KIND_F32 ? (16 * (D / 64) * 64) / kThreads : 4;
  using KReg = typename std::conditional<KIND == KIND_F32 || KIND == KIND_BF16, u32x4, u32x2>::type;
  KReg kr[KCH];
  u32x4 vf[KIND == KIND_F32 ? VCH : 1];
  typename VRawT<KIND == KIND_F32 ? KIND_BF16 : KIND, MD>::T vraw[KIND == KIND_F32 ? 1 : 4];
  float ksc, vsc;   // fp8: the staged tile's K and V scales (per-(page, head) mode)

  // global -> registers for the given tile.  Thread t stages K chunks
  // c = i * 256 + t (lane c % 64 of operand (mb, ks) = c / 64, a row of the
  // tile: key 16 mb + lane % 16) and V rows 32 ks2 + 16 half + 4 (lane / 16) + j.
  // FAST: `page` is the tile's physical page, from the caller's page window.
  // WITH_K = false: V only (K goes straight to LDS)
  template <bool WITH_K = true>
  __device__ __forceinline__ void load(const KParams& p, const SeqCtx& s, int tile, int page) {
    Tile<C::ELT, FAST> t;
    // the tile's scales travel with its data, so the step that uses them
    // does not wait on a dependent page-table and scale lookup
    if constexpr (FAST) {
      t.init_at_page(p, s, tile, page);
      if constexpr (KIND == KIND_F8) ksc = kscale_at_page<KIND>(p, s, page, &vsc);
    } else {
      t.init(p, s, tile);
      if constexpr (KIND == KIND_F8) ksc = kscale_of<KIND>(p, s, t.J0, &vsc);
    }
    const int tid = threadIdx.x;
    const int ln = tid & 63, m = ln & 15, hh = ln >> 4;
    const bool full = t.nvalid == kUnitKeys;
#pragma unroll
    for (int i = 0; i < (WITH_K ? KCH : 0); ++i) {
      const int mk = (i * kThreads + tid) >> 6;            // uniform per wave
      int mb, col;                                          // col: byte offset in the row
      if constexpr (KIND == KIND_F32) {
        mb = mk / (D / 16);
        col = (16 * (mk % (D / 16)) + 4 * hh) * 4;
      } else {
        mb = mk / C::KSQ;
        col = (32 * (mk % C::KSQ) + 8 * hh) * C::ELT;
      }
      const char* row;
      if constexpr (FAST) {
        row = full ? t.kb + 16 * mb * t.kss + ((uint32_t)m * t.kss + col)
                   : t.kb + ((uint32_t)min(16 * mb + m, t.nvalid - 1) * t.kss + col);
      } else {
        row = t.krow(p, s, 16 * mb + m) + col;
      }
      kr[i] = *reinterpret_cast<const KReg*>(row);
    }
    if constexpr (KIND == KIND_F32) {
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        const int grp = (i * kThreads + tid) >> 6;           // (mb * 4 + j) * (D / 64) + gd, uniform per wave
        const int gd = grp % (D / 64), mbj = grp / (D / 64);
        const int mb = mbj >> 2, j = mbj & 3;
        const int kt = 16 * mb + 4 * hh + j;
        const char* row;
        if constexpr (FAST) row = t.vb + (uint32_t)(full ? kt : min(kt, t.nvalid - 1)) * t.vss;
        else row = t.vrow(p, s, kt);
        vf[i] = *reinterpret_cast<const u32x4*>(row + (64 * gd + 4 * m) * 4);
      }
    } else {
      // thread -> (ks2, lane_t, half); 4 rows j = 0..3
      const int task = tid >> 1, half = tid & 1;
      const int ks2 = task >> 6, lt = task & 63;
      const int mm = lt & 15, h2 = lt >> 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kt = 32 * ks2 + 16 * half + 4 * h2 + j;
        const char* row;
        if constexpr (FAST) {
          row = full ? t.vb + (32 * ks2 + j) * t.vss + ((uint32_t)(16 * half + 4 * h2) * t.vss + MD * mm * C::ELT)
                     : t.vb + ((uint32_t)min(kt, t.nvalid - 1) * t.vss + MD * mm * C::ELT);
          vraw[j] = load_v_raw<KIND, MD>(row, 0);
        } else {
          vraw[j] = load_v_raw<KIND, MD>(t.vrow(p, s, kt), MD * mm);
        }
      }
    }
  }

  // registers -> LDS buffer
  template <bool WITH_K = true>
  __device__ __forceinline__ void store(char* kbuf, char* vbuf) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < (WITH_K ? KCH : 0); ++i) {
      const int c = i * kThreads + tid;
      *reinterpret_cast<KReg*>(kbuf + c * sizeof(KReg)) = kr[i];
    }
    if constexpr (KIND == KIND_F32) {
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        const int c = i * kThreads + tid;
        *reinterpret_cast<u32x4*>(vbuf + c * 16) = vf[i];
      }
    } else {
      const int task = tid >> 1, half = tid & 1;
      const int ks2 = task >> 6, ln = task & 63;
      unsigned vb[4][MD / 2];
#pragma unroll
      for (int j = 0; j < 4; ++j) v_words<KIND, MD>(vraw[j], vb[j]);
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const unsigned a0 = vb[0][md >> 1], a1 = vb[1][md >> 1], a2 = vb[2][md >> 1], a3 = vb[3][md >> 1];
        u32x2 w;
        if (md & 1) {
          w[0] = (a0 >> 16) | (a1 & 0xFFFF0000u);
          w[1] = (a2 >> 16) | (a3 & 0xFFFF0000u);
        } else {
          w[0] = (a0 & 0xFFFFu) | (a1 << 16);
          w[1] = (a2 & 0xFFFFu) | (a3 << 16);
        }
        *reinterpret_cast<u32x2*>(vbuf + ((ks2 * MD + md) * 64 + ln) * 16 + 8 * half) = w;
      }
    }
  }
};

// bf16, d = 128, one page per tile: K and V go straight from HBM into LDS
// (buffer_load ... lds), no staging registers.  K operand (mb, ks) = mk lands
// lane-linearly at kbuf + 1 KiB * mk, which is MFMA operand order.  V rows
// 4 r4 .. 4 r4 + 3 land at vbuf + 1 KiB * r4, row-major with row r's 16-byte
// chunk q stored in slot q ^ 2 (r % 8), so the transpose reads of a V^T
// operand (16 rows x 32 bytes) spread over all LDS banks.
struct DirectStage {
  // Per segment: the sequence's K/V bases for kv head g, byte strides, and a
  // 64-entry window of its page table held one entry per lane (a tile's page
  // is then a register read, not a dependent scalar load).
  const char* kbase;
  const char* vbase;
  uint64_t ksp, vsp;          // bytes between pages
  uint32_t kss, vss;          // bytes between slots
  const int32_t* bt_row;
  int pbase, vpage0, vpage1;  // page-table entries pbase + lane and pbase + 64 + lane
  int cur_b, cur_g;
  int page_shift, max_pages, num_pages, page_mask;   // held (see held())
  // per lane: constant parts of the load offsets
  uint32_t k_col, v_col;      // byte column within a row
  int k_row0, v_row0;         // row of load i = 0 (K: + 16 i, V: + 16 i)
  uint32_t k_lane, v_lane;    // byte offsets of the lane's rows for load i = 0
  uint32_t k8_lane;           // fp8 K (see issue_k8): row m, byte 16 hh of a 64-byte chunk
  uint32_t v8_lane;           // fp8 V (see issue_v8): row lane / 8, bytes 16 (lane % 8) ..
  // Segment-constant addressing (SEG; the host selects it only where every
  // byte of the K and of the V cache lies within 2^31 of its head's base):
  // one buffer resource per sequence and kv head, a tile's page and slot as
  // one 32-bit scalar offset, and every DMA's row offset held per lane, so a
  // tile costs a page lookup and two scalar multiplies.
  __amdgpu_buffer_rsrc_t krs_seg, vrs_seg;
  uint32_t ktoff, vtoff;      // the prepared tile's byte offsets from kbase / vbase
  uint32_t ko[4], vo[4];      // per lane: offsets of DMA i (K) and 4 + i (V) within a tile
  uint32_t k8o[2], v8o[2];    // per lane: offsets of the fp8 DMAs (issue_k8, issue_v8)

  // (re)point at sequence s.b, kv head s.g; the page window survives while the
  // sequence stays the same
  // ELT: bytes per K/V element (the direct loads are bf16; other kinds use
  // only the page window)
  template <int ELT = 2, bool SEG = false>
  __device__ __forceinline__ void init(const KParams& p, const SeqCtx& s) {
    if (s.b == cur_b && s.g == cur_g) return;
    if (s.b != cur_b) pbase = -(1 << 30);
    cur_b = s.b;
    cur_g = s.g;
    page_shift = held(p.page_shift);
    max_pages = held(p.max_pages);
    num_pages = held(p.num_pages);
    page_mask = held(p.page_size - 1);
    kbase = wave_uniform(reinterpret_cast<const char*>(p.k) + (int64_t)s.g * p.k_sh * ELT);
    vbase = wave_uniform(reinterpret_cast<const char*>(p.v) + (int64_t)s.g * p.v_sh * ELT);
    ksp = (uint64_t)p.k_sp * ELT;
    vsp = (uint64_t)p.v_sp * ELT;
    kss = (uint32_t)(p.k_ss * ELT);
    vss = (uint32_t)(p.v_ss * ELT);
    bt_row = s.bt_row;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, hh = lane >> 4;
    k_row0 = m;
    k_col = 64u * wave + 16u * hh;                      // K-step ks = wave, dims 32 ks + 8 hh
    const int rl = lane >> 4, sl = lane & 15;
    v_row0 = 4 * wave + rl;                             // row 16 i + 4 wave + rl
    v_col = 16u * (sl ^ (2 * (v_row0 & 7)));             // swizzled 16-byte column (row & 7 is i-invariant)
    k_lane = (uint32_t)k_row0 * kss + k_col;
    v_lane = (uint32_t)v_row0 * vss + v_col;
    k8_lane = (uint32_t)m * kss + 16u * hh;
    v8_lane = (uint32_t)(lane >> 3) * vss + 16u * (lane & 7);
    if constexpr (SEG) {
      krs_seg = tile_rsrc(kbase);
      vrs_seg = tile_rsrc(vbase);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ko[i] = k_lane + (uint32_t)(16 * i) * kss;
        vo[i] = v_lane + (uint32_t)(16 * i) * vss;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        k8o[i] = k8_lane + (uint32_t)(16 * wave) * kss + 64u * i;
        v8o[i] = v8_lane + (uint32_t)(16 * wave + 8 * i) * vss;
      }
    }
  }

  __device__ __forceinline__ int page_of_tile(const KParams& p, int J0) {
    const int idx = J0 >> page_shift;
    if ((unsigned)(idx - pbase) >= 128u) {               // refill the window (rare)
      pbase = idx;
      const int l = (int)(threadIdx.x & 63);
      int v0 = bt_row[min(idx + l, max_pages - 1)];
      int v1 = bt_row[min(idx + 64 + l, max_pages - 1)];
      asm volatile("" : "+v"(v0), "+v"(v1));           // complete the loads here
      vpage0 = v0;
      vpage1 = v1;
    }
    const int i = idx - pbase;
    const int w0 = __builtin_amdgcn_readlane(vpage0, i & 63), w1 = __builtin_amdgcn_readlane(vpage1, i & 63);
    int page = idx < max_pages ? (i < 64 ? w0 : w1) : -1;
    if ((unsigned)page >= (unsigned)num_pages) {
      p.hdr[H_ERROR] = E_PAGE;
      page = 0;
    }
    return page;
  }

  // K in MFMA-operand order at kbuf + 1024 (4 mb + ks); V row-major, 16-byte
  // columns swizzled by row, at vbuf.  Rows past the sequence end re-read its
  // last key (finite values; their scores are masked).
  const char* pk_b;
  const char* pv_b;
  __amdgpu_buffer_rsrc_t krs, vrs;  // the prepared tile's K and V rows (buffer resources)
  int pnvalid;
  int ppage;                  // physical page of the prepared tile
  // The addresses of one tile's DMAs; issue(i) then starts DMA i of 8 (K rows
  // for i < 4, V rows after).  A DMA holds its wave until the address unit
  // takes it, so the tile loop spreads the eight over its QK MFMAs.
  template <bool SEG = false>
  __device__ __forceinline__ void prep(const KParams& p, const SeqCtx& s, int tile) {
    const int J0 = wave_uniform(tile) * kUnitKeys;     // scalar: the tile may arrive in a VGPR
    const int page = page_of_tile(p, J0);
    const uint32_t slot = (uint32_t)(J0 & page_mask);
    // scalar arithmetic throughout (a stride left in a VGPR would put the
    // products on the VALU and read them back)
    const uint32_t kss_s = (uint32_t)__builtin_amdgcn_readfirstlane((int)kss);
    const uint32_t vss_s = (uint32_t)__builtin_amdgcn_readfirstlane((int)vss);
    if constexpr (SEG) {
      ktoff = (uint32_t)wave_uniform((int)((uint32_t)page * (uint32_t)uniform_u64(ksp) + slot * kss_s));
      vtoff = (uint32_t)wave_uniform((int)((uint32_t)page * (uint32_t)uniform_u64(vsp) + slot * vss_s));
      pnvalid = min(kUnitKeys, s.ctx - J0);
      ppage = page;
      return;
    }
    pk_b = wave_uniform(wave_uniform(kbase) + (uint64_t)page * uniform_u64(ksp) + slot * kss_s);
    pv_b = wave_uniform(wave_uniform(vbase) + (uint64_t)page * uniform_u64(vsp) + slot * vss_s);
    krs = tile_rsrc(pk_b);
    vrs = tile_rsrc(pv_b);
    pnvalid = min(kUnitKeys, s.ctx - J0);
    ppage = page;
  }
  // The tile lies in one page, so rows past the sequence end are still cache
  // memory: they are read as they are, their V rows (and in the lean build,
  // which masks by an additive bias, their K rows) are zeroed once landed
  // (zero_tail), and their scores are masked, so no garbage (NaN included)
  // reaches a score or P V.  Row 16 i of a load moves the scalar base only.
  // fp8, d = 128: the K tile straight to LDS in the operand order of the
  // 16x16x128 MFMA with each lane's 32 bytes taken as two 16-byte chunks:
  // chunk c of operand mb (rows 16 mb + m, bytes 64 c + 16 hh) lands
  // lane-linearly at kbuf + 1 KiB (2 mb + c).  Wave w loads operand mb = w.
  template <bool SEG = false>
  __device__ __forceinline__ void issue_k8(int c, char* kbuf) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (SEG) {
      bload16_lds(krs_seg, kbuf + 1024 * (2 * wave + c), k8o[c], ktoff);
      return;
    }
    const uint32_t kss_s = (uint32_t)__builtin_amdgcn_readfirstlane((int)kss);
    bload16_lds(krs, kbuf + 1024 * (2 * wave + c), k8_lane, (uint32_t)(16 * wave) * kss_s + 64u * c);
  }
  // fp8, d = 128: wave w's V rows 16 w + 8 i + lane / 8 (i = 0, 1), 128 bytes
  // each, lane-linearly into the staging block at v8buf + 1 KiB (2 w + i).
  // Only wave w reads them back (widen_v8), so the wave's own wait orders
  // them; the block needs no second buffer.
  template <bool SEG = false>
  __device__ __forceinline__ void issue_v8(int i, char* v8buf) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (SEG) {
      bload16_lds(vrs_seg, v8buf + 1024 * (2 * wave + i), v8o[i], vtoff);
      return;
    }
    const uint32_t vss_s = (uint32_t)__builtin_amdgcn_readfirstlane((int)vss);
    bload16_lds(vrs, v8buf + 1024 * (2 * wave + i), v8_lane, (uint32_t)(16 * wave + 8 * i) * vss_s);
  }
  // After this wave's V DMAs have landed (vmcnt): its 16 rows of fp8 V to
  // bf16 (exact: every E4M3 value is a bf16), written row-major into the V
  // stage with the bf16 direct path's swizzle (16-byte chunk q of row r in
  // slot q ^ 2 (r % 8)).  Rows past the sequence end (the last tile only) are
  // written as zeros, so no garbage (NaN included) reaches P V.  A lane of an
  // odd row takes its two 8-byte halves in the other order, so the 16 lanes of
  // one LDS write (two rows) fill both the even and the odd chunk slots: no
  // bank conflicts (measured 2% faster dense fp8 prefill).
  __device__ __forceinline__ void widen_v8(const char* v8buf, char* vbuf) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * wave + 8 * i + (lane >> 3), q = lane & 7;    // fp8 bytes 16 q .. 16 q + 15 of row r
      const int odd = (lane >> 3) & 1;                              // r & 1
      const char* src = v8buf + 1024 * (2 * wave + i) + 16 * lane;
      const u32x2 f0 = *reinterpret_cast<const u32x2*>(src + 8 * odd);
      const u32x2 f1 = *reinterpret_cast<const u32x2*>(src + 8 * (1 - odd));
      u32x4 raw = u32x4{f0[0], f0[1], f1[0], f1[1]};
      if (pnvalid < kUnitKeys && r >= pnvalid) raw = u32x4{0, 0, 0, 0};
      u32x4 lo, hi;          // bf16 of fp8 bytes 16 q + 8 odd .. + 7 and 16 q + 8 (1 - odd) .. + 7
      lo[0] = f8x2_to_bf16x2(raw[0]);
      lo[1] = f8x2_to_bf16x2<true>(raw[0]);
      lo[2] = f8x2_to_bf16x2(raw[1]);
      lo[3] = f8x2_to_bf16x2<true>(raw[1]);
      hi[0] = f8x2_to_bf16x2(raw[2]);
      hi[1] = f8x2_to_bf16x2<true>(raw[2]);
      hi[2] = f8x2_to_bf16x2(raw[3]);
      hi[3] = f8x2_to_bf16x2<true>(raw[3]);
      char* row = vbuf + 256 * r;
      const int sw = 2 * (r & 7);
      *reinterpret_cast<u32x4*>(row + 16 * ((2 * q + odd) ^ sw)) = lo;
      *reinterpret_cast<u32x4*>(row + 16 * ((2 * q + 1 - odd) ^ sw)) = hi;
    }
  }
  template <bool SEG = false>
  __device__ __forceinline__ void issue(int i, char* kbuf, char* vbuf) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (SEG) {
      if (i < 4) bload16_lds(krs_seg, kbuf + 1024 * (4 * i + wave), ko[i], ktoff);
      else bload16_lds(vrs_seg, vbuf + 1024 * (4 * (i - 4) + wave), vo[i - 4], vtoff);
      return;
    }
    const uint32_t kss_s = (uint32_t)__builtin_amdgcn_readfirstlane((int)kss);
    const uint32_t vss_s = (uint32_t)__builtin_amdgcn_readfirstlane((int)vss);
    if (i < 4) bload16_lds(krs, kbuf + 1024 * (4 * i + wave), k_lane, (uint32_t)(16 * i) * kss_s);
    else bload16_lds(vrs, vbuf + 1024 * (4 * (i - 4) + wave), v_lane, (uint32_t)(16 * (i - 4)) * vss_s);
  }
  // Segment-constant addressing with the tile offsets given: DMA i of a K tile
  // (i < 4, offset kto) or of a V tile (i >= 4, offset vto), so that one step
  // can load K and V of different tiles
  __device__ __forceinline__ void issue_at(int i, char* kbuf, char* vbuf, uint32_t kto, uint32_t vto) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (i < 4) bload16_lds(krs_seg, kbuf + 1024 * (4 * i + wave), ko[i], kto);
    else bload16_lds(vrs_seg, vbuf + 1024 * (4 * (i - 4) + wave), vo[i - 4], vto);
  }
  // after this wave's DMAs into kbuf and vbuf have landed (vmcnt): zero the
  // V rows (and with K, the K rows) it loaded past the sequence end; every
  // lane clears the 16 bytes it wrote (K load i holds rows 16 i + lane % 16,
  // see issue).  nvalid: the tile's valid keys (default: the prepared tile's)
  template <bool K>
  __device__ __forceinline__ void zero_tail(char* kbuf, char* vbuf) { zero_tail_n<K>(kbuf, vbuf, pnvalid); }
  template <bool K>
  __device__ __forceinline__ void zero_tail_n(char* kbuf, char* vbuf, int nvalid) {
    if (nvalid >= kUnitKeys) return;                      // uniform: only a sequence's last tile
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (K && k_row0 + 16 * i >= nvalid)
        *reinterpret_cast<u32x4*>(kbuf + 1024 * (4 * i + wave) + 16 * lane) = u32x4{0, 0, 0, 0};
      if (v_row0 + 16 * i >= nvalid)
        *reinterpret_cast<u32x4*>(vbuf + 1024 * (4 * i + wave) + 16 * lane) = u32x4{0, 0, 0, 0};
    }
  }
  // fp8: the same for the K rows of issue_k8 (wave w: rows 16 w + lane % 16)
  __device__ __forceinline__ void zero_tail_k8(char* kbuf) {
    if (pnvalid >= kUnitKeys) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (16 * wave + (lane & 15) >= pnvalid) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
        *reinterpret_cast<u32x4*>(kbuf + 1024 * (2 * wave + c) + 16 * lane) = u32x4{0, 0, 0, 0};
    }
  }
  template <bool SEG = false>
  __device__ __forceinline__ void load(const KParams& p, const SeqCtx& s, int tile, char* kbuf, char* vbuf) {
    prep<SEG>(p, s, tile);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue<SEG>(i, kbuf, vbuf);
  }
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// A workgroup barrier for LDS only: this wave's LDS writes complete, then the
// barrier, with no wait on vector memory (the fence of __syncthreads would
// drain every DMA still in flight).  The LDS DMAs a barrier must cover are
// waited for explicitly before it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef short i16x4 __attribute__((ext_vector_type(4)));

// V^T operand (ks2, md) of a row-major swizzled V tile by two transpose reads:
// in each 16-lane group h, lane i = 4 k + c points at row 32 ks2 + 4 h + k
// (+16 for slots 4..7), dims 16 md + 4 c; the read hands lane i the dim
// 16 md + i of those 4 rows.  `base0` is the lane's byte offset with md = 0
// (row part + swizzle bits), so the md offset is an XOR on bits 5..7.
// `trx` = the lane's offset with the md XOR applied (below 4096, so adding a
// buffer offset that is a multiple of 4096 commutes with the XOR and folds
// into the instruction's immediate offset).
__device__ __forceinline__ bf16x8 v_operand_tr(const char* smem, uint32_t trx, uint32_t off) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(smem + trx + off));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(smem + trx + off + 4096));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

// LEAN: a build for calls with no block mask and a landmark chunk that is 0 or
// a multiple of 64, where the only landmark a tile can hold is its last key
// (offset 63: accumulator slot (3, 3) of lane group 3), so a fully visible
// tile masks it with one select per row block and the block-mask code is gone;
// its DMAs use the segment-constant addressing of DirectStage (SEG).
template <int KIND, int D, bool FAST, bool LEAN = false>
__device__ PA_SEGMENT_FN void large_segment(uint64_t pk, const QBlock x, int t_lo, int t_hi, int u0,
                                                       int u1, bool final_out, int slot, DirectStage& ds) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const KParams& p = kparams_at(pk);
  using C = Cfg<KIND, D>;
  constexpr int MD = C::MD;
  constexpr int NB = 2;
  constexpr bool DIRECT = KIND == KIND_BF16 && D == 128 && FAST;
  // fp8, d = 128, one page per tile: K straight to LDS in the 16x16x128
  // operand order (issue_k8; Q takes K's chunk order); V straight to an LDS
  // staging block (issue_v8), each wave widening its own rows to bf16 into the
  // V stage (widen_v8), so PV reads bf16 V^T operands as the bf16 path does
  constexpr bool DKF8 = KIND == KIND_F8 && D == 128 && FAST;
  // PV operands by transpose reads from a row-major bf16 V stage
  constexpr bool TRV = DIRECT || DKF8;
  // The lean bf16 build keeps three K stages and two V stages: a step issues
  // the next tile's V (first) and the K of the tile after it, so both have
  // more than a tile of QK, softmax and PV to land (the V DMAs go out in the
  // first half of the QK loop).  The K stage rotates at run time (one base
  // per tile for its reads); the V stage alternates with the step's parity.
  constexpr bool K3 = LEAN && DIRECT;
  // The lean fp8 build widens a tile's V at the start of its own step (the
  // conversions run beside the QK MFMAs), with an LDS barrier before PV
  // instead of the widening at the end of the previous step.
  constexpr bool WD = LEAN && DKF8;
  int ks = 0;                         // K3: the current tile's K stage
  uint32_t vt_next = 0;               // K3: V offset of the tile after the current one
  int nv_next = kUnitKeys;            //      and its valid keys
  char* const v8buf = smem + 2 * C::K_TILE;         // DKF8: fp8 V staging (single)
  // Row sums of P stay on the VALU in fp32: an MFMA sum of the bf16 P operand
  // carries its rounding (up to 2^-9 on the largest term, which under the lazy
  // rescale is no longer exactly 1) straight into the LSE.
  constexpr bool MSUM = false;
  // the wave index is the same in every lane: scalar, so that per-wave bounds
  // and the per-tile tests built on them are scalar branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, h = lane >> 4;
  short* list = reinterpret_cast<short*>(smem + Lds<KIND, D, FAST>::DYN - kMaskListCap * 2);
  SeqCtx s{x.b, x.g, x.ctx, t_lo, p.bt + (int64_t)x.b * p.bt_stride};
  // transpose-read lane offsets (see v_operand_tr), relative to a V buffer
  const int trk = n >> 2, trc = n & 3;
  const uint32_t tr_lane = (uint32_t)(4 * h + trk) * 256u + 32u * ((4 * h + trk) & 7) + 16u * (trc >> 1) + 8u * (trc & 1);
  uint32_t trx[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) trx[md] = tr_lane ^ (32u * md);

  // this lane's two rows
  typename QKOpT<KIND>::T qB[NB][C::KSQ];
  RowMask rm[NB];
  int rowi[NB];
  bool rok[NB];
  int bm_head[NB];
  int pos_min = 0x7fffffff, left_max = 0;
  const bool wave_live = 32 * wave < x.rows;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = 32 * wave + 16 * nb + n;
    rok[nb] = r < x.rows;
    rowi[nb] = rok[nb] ? r : 0;
    const int tok = x.q0 + x.t0 + rowi[nb] / p.G, head = x.g * p.G + rowi[nb] % p.G;
    const char* qrow = rok[nb] ? reinterpret_cast<const char*>(p.q) + (tok * p.q_st + head * p.q_sh) * C::ELT
                               : nullptr;
    if constexpr (DKF8) {
      // bytes 16 h .. 16 h + 15 and 64 + 16 h .. 79 + 16 h of the row, as issue_k8 lays K out
      const u32x4 c0 = qrow ? *reinterpret_cast<const u32x4*>(qrow + 16 * h) : u32x4{0, 0, 0, 0};
      const u32x4 c1 = qrow ? *reinterpret_cast<const u32x4*>(qrow + 64 + 16 * h) : u32x4{0, 0, 0, 0};
      qB[nb][0] = __builtin_bit_cast(long, u32x2{c0[0], c0[1]});
      qB[nb][1] = __builtin_bit_cast(long, u32x2{c0[2], c0[3]});
      qB[nb][2] = __builtin_bit_cast(long, u32x2{c1[0], c1[1]});
      qB[nb][3] = __builtin_bit_cast(long, u32x2{c1[2], c1[3]});
    } else {
      load_qk_row<KIND, D>(qrow, h, qB[nb]);
    }
    rm[nb].pos = x.ctx - x.ql + x.t0 + rowi[nb] / p.G;
    rm[nb].left = p.window > 0 ? window_left(p, rm[nb].pos) : 0;
    rm[nb].bit = true;
    rm[nb].qs = qscale_of<KIND>(p, tok, head);
    bm_head[nb] = p.bm && p.bm_heads != 1 ? head : 0;
  }
  if (wave_live) {
    // bounds over this wave's valid rows (uniform across the wave)
    const int r_lo = 32 * wave, r_hi = min(x.rows, 32 * wave + 32) - 1;
    pos_min = x.ctx - x.ql + x.t0 + r_lo / p.G;
    const int pos_hi_w = x.ctx - x.ql + x.t0 + r_hi / p.G;
    left_max = p.window > 0 ? window_left(p, pos_hi_w) : 0;
  }

  TileParams tp = TileParams::held_of(p);
  if constexpr (LEAN) tp.has_bm = 0;
  WaveState<KIND, D, NB> st;
  st.init();
  Stage<KIND, D, FAST> stg;
  stg.ksc = stg.vsc = 1.f;
  float cur_ksc = 1.f, cur_vsc = 1.f;              // scales of the tile in the current stage
  // fp8: a V scale per (page, kv head) goes into P tile by tile; the one V
  // scale of a tensor multiplies O once, in the epilogue
  bool v_per_tile = false;
  float v_out = 1.f;
  if constexpr (DKF8) {
    v_per_tile = held((p.scale_mode & 3) == 2 ? 1 : 0) != 0;
    v_out = v_per_tile ? 1.f : p.v_scale[0];
  }
  if constexpr (FAST) ds.init<C::ELT, LEAN>(p, s);       // keeps its page window while the sequence stays

  for (int c0 = u0; c0 < u1; c0 += kMaskListCap) {
    const int cn = min(kMaskListCap, u1 - c0);
    if (tp.has_bm) build_tile_list(p, x, t_lo, t_hi, c0, cn, list);
    auto tile_of = [&](int u) {   // wave-uniform: keeps tile addressing in scalar registers
      return __builtin_amdgcn_readfirstlane(tp.has_bm ? (int)list[u - c0] : t_lo + u);
    };
    if constexpr (K3) {
      // tile c0's K and V, landed and tail-zeroed; then the K of tile c0 + 1
      // goes out and its V offsets are kept for the first step
      ks = 0;
      ds.load<LEAN>(p, s, tile_of(c0), smem, vstage<true>(0));
      wait_vmem();
      ds.zero_tail<true>(smem, vstage<true>(0));
      ds.prep<LEAN>(p, s, tile_of(min(c0 + 1, c0 + cn - 1)));
      vt_next = ds.vtoff;
      nv_next = ds.pnvalid;
#pragma unroll
      for (int i = 0; i < 4; ++i) ds.issue_at(i, smem + C::K_TILE, nullptr, ds.ktoff, 0);
    } else if constexpr (DIRECT) {
      ds.load<LEAN>(p, s, tile_of(c0), smem, vstage<true>(0));
      wait_vmem();
      ds.zero_tail<LEAN>(smem, vstage<true>(0));
    } else if constexpr (DKF8) {
      ds.prep<LEAN>(p, s, tile_of(c0));
      ds.issue_k8<LEAN>(0, smem);
      ds.issue_k8<LEAN>(1, smem);
      ds.issue_v8<LEAN>(0, v8buf);
      ds.issue_v8<LEAN>(1, v8buf);
      cur_ksc = kscale_at_page<KIND>(p, s, ds.ppage, &cur_vsc);
      wait_vmem();
      if constexpr (LEAN) ds.zero_tail_k8(smem);
      if constexpr (!WD) ds.widen_v8(v8buf, vstage<true>(0));
    } else {
      stg.load(p, s, tile_of(c0), FAST ? ds.page_of_tile(p, tile_of(c0) * kUnitKeys) : -1);
      stg.store(smem, smem + C::K_TILE);
      cur_ksc = stg.ksc;
      cur_vsc = stg.vsc;
    }
    if constexpr (K3) lds_barrier();
    else __syncthreads();
    // one tile; BUF (a compile-time 0 / 1) selects the stage it reads, so every
    // LDS address is a lane register plus an immediate offset
    auto step = [&](int u, auto buf_c) {
      constexpr int buf = decltype(buf_c)::value;
      char* kbuf = K3 ? smem + ks * C::K_TILE : TRV ? smem + buf * C::K_TILE : smem + buf * C::STAGE;
      char* vbuf = kbuf + C::K_TILE;
      const bool more = u + 1 < c0 + cn;
      const int ks2 = ks == 0 ? 2 : ks - 1;             // K3: the stage two tiles ahead ((ks + 2) % 3)
      char* nkb = K3 ? smem + ks2 * C::K_TILE : smem + (buf ^ 1) * C::K_TILE;
      char* nvb = nullptr;
      uint32_t vt1 = 0, kt2 = 0;                       // K3: V offset of tile u + 1, K offset of tile u + 2
      int nv1 = kUnitKeys;
      float nksc = 1.f, nvsc = 1.f;                    // DKF8: scales of the next tile
      if constexpr (DKF8) {
        if constexpr (WD) {
          // this tile's V (landed at the end of the previous step) to bf16
          // into its V stage; the staging block's reads complete before the
          // next tile's V DMAs below may write it
          ds.widen_v8(v8buf, vstage<true>(buf));
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        // the next tile's K and V go out before the QK MFMAs (a chunk's last
        // step re-loads its own tile into the idle stage, as the bf16 path)
        nvb = vstage<true>(buf ^ 1);
        ds.prep<LEAN>(p, s, tile_of(more ? u + 1 : u));
        ds.issue_k8<LEAN>(0, nkb);
        ds.issue_k8<LEAN>(1, nkb);
        ds.issue_v8<LEAN>(0, v8buf);
        ds.issue_v8<LEAN>(1, v8buf);
        nksc = kscale_at_page<KIND>(p, s, ds.ppage, &nvsc);
      } else if constexpr (K3) {
        // the V of tile u + 1 and the K of tile u + 2 go out between the QK
        // MFMAs below, V first (past the chunk's end a step re-loads its
        // last tile into an idle stage)
        nvb = vstage<true>(buf ^ 1);
        vt1 = vt_next;
        nv1 = nv_next;
        ds.prep<LEAN>(p, s, tile_of(min(u + 2, c0 + cn - 1)));
        kt2 = ds.ktoff;
        vt_next = ds.vtoff;
        nv_next = ds.pnvalid;
        if (!wave_live) {                               // a wave with no rows still loads its share
#pragma unroll
          for (int i = 0; i < 8; ++i) ds.issue_at(i < 4 ? 4 + i : i - 4, nkb, nvb, kt2, vt1);
        }
      } else if constexpr (DIRECT) {
        // the next tile's DMAs go out between the QK MFMAs below (the last
        // step of a chunk re-loads its own tile into the idle stage)
        nvb = vstage<true>(buf ^ 1);
        ds.prep<LEAN>(p, s, tile_of(more ? u + 1 : u));
        if (!wave_live) {                               // a wave with no rows still loads its share
#pragma unroll
          for (int i = 0; i < 8; ++i) ds.issue<LEAN>(i, nkb, nvb);
        }
      } else if (more) {
        stg.load(p, s, tile_of(u + 1), FAST ? ds.page_of_tile(p, tile_of(u + 1) * kUnitKeys) : -1);
      }
      __builtin_amdgcn_sched_barrier(0);
      const int tile = tile_of(u);
      const int J0 = tile * kUnitKeys;
      if (wave_live) {
        float vsc = 1.f, ksc = 1.f;
        if constexpr (KIND == KIND_F8) {
          ksc = cur_ksc;
          vsc = cur_vsc;
        }
        float cs = tp.sm_log2;
        if constexpr (KIND == KIND_F8) cs *= ksc;
        if (tp.has_bm) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int kt = J0 / p.bm_tile, qt = rm[nb].pos / p.bm_tile;
            rm[nb].bit = kt < p.bm_nk && qt < p.bm_nq &&
                         p.bm[x.b * p.bm_sb + bm_head[nb] * p.bm_sh + qt * p.bm_sq + kt * p.bm_sk] != 0;
          }
        }
        const int nvalid = min(kUnitKeys, x.ctx - J0);
        // LEAN: key J0 + 63 is a landmark when (J0 + 64) is a multiple of the chunk
        const bool lm63 = LEAN && tp.landmark > 0 &&
                          (tp.landmark == kUnitKeys || (J0 + kUnitKeys) % tp.landmark == 0);
        const uint64_t lmk = LEAN ? (lm63 ? uint64_t(1) << (kUnitKeys - 1) : 0) : landmark_bits(tp, J0);
        const bool full = unit_is_full(tp, J0, nvalid, pos_min, left_max);
        // S^T = K Q^T.  The lean build takes a tile's mask as the initial
        // accumulator of its QK MFMAs (0 where a score is visible, -inf where
        // masked), so masked and unmasked tiles leave their scores in the same
        // registers with no select after the products (a select there makes
        // the compiler copy all 32 scores on every unmasked tile).  Keys past
        // the sequence end are zeros in LDS (zero_tail), so a masked score is
        // -inf, never NaN.  The other builds select after the products: the
        // 32 bias registers would push them into spills.
        f32x4 sc[NB][4];
        if constexpr (!LEAN) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) sc[nb][mb] = f32x4{0, 0, 0, 0};
        }
        if constexpr (KIND == KIND_F32) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int cc = 0; cc < D / 16; ++cc) {
              const f32x4 ka = *reinterpret_cast<const f32x4*>(kbuf + ((mb * (D / 16) + cc) * 64 + lane) * 16);
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) sc[nb][mb] = mfma_qk(ka[i], qB[nb][4 * cc + i], sc[nb][mb]);
            }
        } else {
          // K operand reads.  fp8: the first operand goes out ahead of the
          // branch on the tile's mask below, so its latency does not wait on
          // it (bf16 keeps its first reads in the branches: eight operands
          // held across the mask's bias would spill)
          auto kread4 = [&](int mb) -> i32x8 {            // fp8, d = 128: operand mb
            if constexpr (DKF8) {
              const u32x4 a = *reinterpret_cast<const u32x4*>(kbuf + 1024 * (2 * mb) + 16 * lane);
              const u32x4 b = *reinterpret_cast<const u32x4*>(kbuf + 1024 * (2 * mb + 1) + 16 * lane);
              return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
            } else {
              const char* at = kbuf + (mb * 4 * 64 + lane) * 8;
              return cat4(*reinterpret_cast<const long*>(at), *reinterpret_cast<const long*>(at + 512),
                          *reinterpret_cast<const long*>(at + 1024), *reinterpret_cast<const long*>(at + 1536));
            }
          };
          using KT = typename QKOpT<KIND>::T;
          auto kread = [&](int i) -> KT {                 // other kinds: operand i
            if constexpr (KIND == KIND_BF16)
              return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kbuf + (i * 64 + lane) * 16));
            else
              return *reinterpret_cast<const long*>(kbuf + (i * 64 + lane) * 8);
          };
          // K-step outermost: the eight accumulators of a step are independent,
          // so no MFMA waits on the result of the one just issued
          constexpr int NK = 4 * C::KSQ, KDEP = 8;
          auto kix = [](int i) { return (i % 4) * C::KSQ + i / 4; };
          constexpr bool QK128 = KIND == KIND_F8 && D == 128;
          i32x8 kc0;
          if constexpr (QK128) kc0 = kread4(0);
          // init(nb, mb): the lean build's initial accumulator of row-block nb,
          // key block mb (the other builds start from the zeros above)
          auto qk = [&](auto init) {
            if constexpr (QK128) {
              // one 16x16x128 MFMA per (mb, nb); the next mb's four K operands
              // are read while this mb's MFMAs run
              i32x8 qc[NB];
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) qc[nb] = cat4(qB[nb][0], qB[nb][1], qB[nb][2], qB[nb][3]);
              i32x8 kc = kc0;
#pragma unroll
              for (int mb = 0; mb < 4; ++mb) {
                const i32x8 ka = kc;
                if (mb + 1 < 4) kc = kread4(mb + 1);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) sc[nb][mb] = mfma_qk128(ka, qc[nb], LEAN ? init(nb, mb) : sc[nb][mb]);
              }
            } else {
              // K operands stream from LDS KDEP reads ahead of the MFMAs that
              // use them (the schedule groups below keep that order), so the
              // reads' latency hides behind the matrix work instead of
              // stalling each MFMA
              KT kr[KDEP];
#pragma unroll
              for (int i = 0; i < KDEP; ++i) kr[i] = kread(kix(i));
              __builtin_amdgcn_sched_group_barrier(0x100, KDEP, 0);
#pragma unroll
              for (int i = 0; i < NK; ++i) {
                const KT ka = kr[i % KDEP];
                if (i + KDEP < NK) kr[i % KDEP] = kread(kix(i + KDEP));
                const int mb = i % 4, ks = i / 4;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) sc[nb][mb] = mfma_qk(ka, qB[nb][ks], LEAN && ks == 0 ? init(nb, mb) : sc[nb][mb]);
                if constexpr (K3) {
                  if (i % 2 == 1) ds.issue_at(i / 2 < 4 ? 4 + i / 2 : i / 2 - 4, nkb, nvb, kt2, vt1);
                } else if constexpr (DIRECT) {
                  if (i % 2 == 1) ds.issue<LEAN>(i / 2, nkb, nvb);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
                if (i + KDEP < NK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if constexpr (DIRECT) { if (i % 2 == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); }
              }
            }
          };
          const auto zero_init = [](int, int) { return f32x4{0, 0, 0, 0}; };
          if (!LEAN || (full && lmk == 0)) {
            qk(zero_init);
          } else if (full) {
            // LEAN: the only landmark of a full tile is key 63, slot (3, 3) of
            // lane group 3
            const f32x4 lmb = f32x4{0, 0, 0, h == 3 ? kNegInf : 0.f};
            qk([&](int, int mb) { return mb == 3 ? lmb : f32x4{0, 0, 0, 0}; });
          } else {
            // a tile that is not full; the lane bitmaps are built from an
            // opaque copy of the landmark bits, so none of that work is
            // hoisted onto the tiles that need no mask at all
            uint64_t lm = lmk;
            asm volatile("" : "+s"(lm));
            f32x4 bias[NB][4];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              ElemMask em;
              em.init(tp, rm[nb], J0, nvalid, lm, h);
              mask_bias(bias[nb], em, h);
            }
            qk([&](int nb, int mb) { return bias[nb][mb]; });
          }
        }
        // the softmax (VALU work) runs at raised wave priority, so on a SIMD
        // shared with the other workgroup's wave it goes ahead of that wave's
        // matrix work instead of queueing behind it (measured faster)
        __builtin_amdgcn_s_setprio(1);
        if constexpr (!LEAN) {
          if (!full || lmk != 0) {
            uint64_t lm = lmk;
            asm volatile("" : "+s"(lm));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              if (!full) {
                ElemMask em;
                em.init(tp, rm[nb], J0, nvalid, lm, h);
                mask_scores(sc[nb], em, h);
              } else {
                mask_landmarks(sc[nb], lm, h);
              }
            }
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          softmax_update<KIND, D, NB, !MSUM>(st, nb, sc[nb], KIND == KIND_F8 ? cs * rm[nb].qs : cs);
        __builtin_amdgcn_s_setprio(0);
        // WD: every wave's widened V rows are in LDS before any PV read (a
        // wave with no rows takes its barrier in the else branch below)
        if constexpr (WD) lds_barrier();
        // O^T += V^T P^T
        if constexpr (KIND == KIND_F32) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int gd = 0; gd < D / 64; ++gd) {
                const f32x4 va = *reinterpret_cast<const f32x4*>(vbuf + ((((mb * 4 + j) * (D / 64)) + gd) * 64 + lane) * 16);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                  for (int nb = 0; nb < NB; ++nb)
                    st.acc[nb][4 * gd + i] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[i], sc[nb][mb][j], st.acc[nb][4 * gd + i], 0, 0, 0);
              }
        } else if constexpr (TRV) {
          // V^T operands by transpose reads, VDEP operands ahead of their MFMAs
          // (ten in the lean fp8 build: measured on MI355X 7% faster than
          // eight, and 1.7% faster than twelve with per-(page, head) scales,
          // equal per tensor; the general builds spill with more than eight)
          constexpr int NV = 2 * MD, VDEP = KIND == KIND_F8 && LEAN ? 10 : 8;
          auto vread = [&](int i) -> bf16x8 {
            return v_operand_tr(vstage<true>(buf), trx[i % MD], (uint32_t)((i / MD) * 8192));
          };
          bf16x8 pb[2][NB];
          // fp8 with one V scale for the tensor: applied to O in the epilogue,
          // not to every P; a V scale per (page, head) changes per tile
          if (KIND != KIND_F8 || v_per_tile) {
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) pb[ks2][nb] = p_operand(sc[nb], ks2, vsc);
          } else {
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) pb[ks2][nb] = p_operand(sc[nb], ks2, 1.f);
          }
          bf16x8 vr[VDEP];
#pragma unroll
          for (int i = 0; i < VDEP; ++i) vr[i] = vread(i);
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * VDEP, 0);
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            const bf16x8 va = vr[i % VDEP];
            if (i + VDEP < NV) vr[i % VDEP] = vread(i + VDEP);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) st.acc[nb][i % MD] = mfma_pv(va, pb[i / MD][nb], st.acc[nb][i % MD]);
            __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
            if (i + VDEP < NV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        } else {
#pragma unroll
          for (int ks2 = 0; ks2 < 2; ++ks2) {
            bf16x8 pb[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) pb[nb] = p_operand(sc[nb], ks2, vsc);
            if constexpr (MSUM) {
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) st.lacc[nb] = mfma_pv(ones_bf16x8(), pb[nb], st.lacc[nb]);
            }
#pragma unroll
            for (int md = 0; md < MD; ++md) {
              const bf16x8 va = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vbuf + ((ks2 * MD + md) * 64 + lane) * 16));
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) st.acc[nb][md] = mfma_pv(va, pb[nb], st.acc[nb][md]);
            }
          }
        }
      } else {
        if constexpr (WD) lds_barrier();
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (K3) {
        // tile u + 1's K (issued a step ago) and V (this step) have landed;
        // the four K DMAs of tile u + 2, issued last, may still be in flight
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        ks = ks == 2 ? 0 : ks + 1;
        ds.zero_tail_n<true>(smem + ks * C::K_TILE, nvb, nv1);
      } else if constexpr (DIRECT) {
        wait_vmem();
        ds.zero_tail<LEAN>(nkb, nvb);
      } else if constexpr (DKF8) {
        wait_vmem();                                     // this wave's K and V DMAs have landed
        if constexpr (LEAN) ds.zero_tail_k8(nkb);
        if constexpr (!WD) ds.widen_v8(v8buf, nvb);
        cur_ksc = nksc;
        cur_vsc = nvsc;
      } else if (more) {
        char* nk = smem + (buf ^ 1) * C::STAGE;
        stg.store(nk, nk + C::K_TILE);
        cur_ksc = stg.ksc;
        cur_vsc = stg.vsc;
      }
      if constexpr (K3) lds_barrier();
      else __syncthreads();
    };
    for (int u = c0; u < c0 + cn; u += 2) {
      step(u, std::integral_constant<int, 0>{});
      if (u + 1 < c0 + cn) step(u + 1, std::integral_constant<int, 1>{});
    }
    // K3: the last step's K DMAs (into an idle stage) land before the stages
    // are reused (the next chunk, or the fused merge's slots)
    if constexpr (K3) wait_vmem();
  }

  // epilogue: per lane row, reduce l over the four lane groups and write
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l = MSUM ? st.lacc[nb][0] : row_sum4(st.lsum[nb]);
    if (!rok[nb]) continue;
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : (DKF8 && !v_per_tile ? v_out : 1.f) / l;
    const float lse = empty ? kNegInf : (st.m2(nb) + log2f(l)) * kLn2;
    write_row<KIND, D, TRV>(p, x, rowi[nb], h, st.acc[nb], inv, lse, final_out, slot);
  }
}

// ---------------------------------------------------------------------------
// static split: item it = (Q-block it / S, split it % S), mapped from the
// workgroup id with no task map ("Triton-TLE rewrite of Tencent HPC-Ops
// Attention", §1.2, the static Split-K variant: a fixed number of splits)
// ---------------------------------------------------------------------------
template <int KIND, int D, bool FAST>
__device__ __forceinline__ void static_items(uint64_t pk) {
  const KParams& p = kparams_at(pk);
  const int S = p.static_S;
  const int n_items = p.B * p.Hkv * S;
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int q = it / S, s = it - q * S;
    QBlock x;
    const int err = static_qblock(p, q, x);
    if (err != E_NONE) {
      if (threadIdx.x == 0) p.hdr[H_ERROR] = err;
      continue;
    }
    if (x.ql == 0) continue;
    const StaticSplit sp = static_split(p, x);
    const int u0 = s * sp.c;
    if (sp.n == 0) {
      // no visible key: split 0 writes the empty rows
      if (s == 0) small_segment<KIND, D, FAST>(pk, x, 0, 0, 0, 0, true, 0);
      continue;
    }
    if (u0 >= sp.n) continue;
    const bool final_out = sp.ns == 1;
    small_segment<KIND, D, FAST>(pk, x, sp.t_lo, sp.t_lo + sp.n - 1, u0, min(sp.n, u0 + sp.c), final_out,
                                 final_out ? 0 : it);
    if (!final_out && p.fused) finish_split<KIND, D>(p, q, x, sp.ns, q * S);
  }
}

// ---------------------------------------------------------------------------
// the persistent kernel
// ---------------------------------------------------------------------------

// PATHS: which Q-block paths the kernel is built with.  kPathsSmall is the
// kernel for batches whose Q-blocks are all small (decode and MTP, and every
// static split); kPathsLarge the one for batches whose Q-blocks are all large
// (prefill chunks, the sliding-window forward).  Each is the same code with
// the other path left out, compiled on its own: sharing one kernel with the
// other path's register demand costs the decode loops 7-13% and the prefill
// loops 2-8% (measured), although their instruction streams come out nearly
// the same.  The small-only kernel reports a large Q-block (E_QLEN_HINT) and
// skips it; the large-only kernel runs the few-row tail Q-blocks of long
// sequences on the 128-row path (Assign rejects short sequences under it).
// kPathsHeads is the kernel for sequence Q-blocks (heads_range only).
// kPathsLean is the large-only kernel with large_segment's LEAN build.
constexpr int kPathsAll = 0, kPathsSmall = 1, kPathsLarge = 2, kPathsHeads = 3, kPathsLean = 4;

template <int KIND, int D, bool FAST, int PATHS>
__global__ __launch_bounds__(kThreads, (Lds<KIND, D, FAST>::OCC)) void attention_kernel(KParams) {
  constexpr bool SMALL = PATHS == kPathsSmall, LARGE = PATHS == kPathsLarge || PATHS == kPathsLean,
                 HEADS = PATHS == kPathsHeads;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const uint64_t pk = kparams_addr();
  const KParams& p = kparams_at(pk);
  if constexpr (SMALL) {
    if (p.static_S > 0) {
      static_items<KIND, D, FAST>(pk);
      return;
    }
  }
  const int U = p.hdr[H_U];
  const WorkerMap wm{p.hdr[H_L], p.hdr[H_L0]};
  const int n_workers = p.hdr[H_NWORKERS];
  if (p.fused) {
    // Q-blocks without a unit (no visible key): their rows, spread over the grid
    const int n_combine = p.hdr[H_NCOMBINE];
    for (int i = blockIdx.x; i < n_combine; i += gridDim.x) {
      const int q = p.combine_list[i];
      if (p.n_splits[q] == 0)
        merge_qblock<D, KIND == KIND_F32>(p, load_qblock(p, q), 0, 0, reinterpret_cast<MergeState*>(smem));
    }
  }
  if (U == 0 || n_workers == 0) return;
  // XCD-aware numbering: consecutive workgroup ids land on different XCDs, so
  // each XCD gets a contiguous block of workers (neighbouring units share K/V
  // in its L2).  The small-Q-block kernel also pairs workers per compute unit:
  // workgroups b and b + grid / 2 run on one unit (two per unit) and become
  // the worker pair (2k, 2k + 1), the first dispatched taking the pair's
  // first (weighted) run.  The general kernel keeps workers r and r + grid / 16
  // on one unit (measured faster for prefill and sliding-window batches).
  int rank = blockIdx.x;
  if ((SMALL || HEADS) && (gridDim.x & 15) == 0) {
    const int half = gridDim.x >> 1, b = blockIdx.x % half;
    rank = 2 * ((b & 7) * (half >> 3) + (b >> 3)) + (blockIdx.x >= half ? 1 : 0);
  } else if (gridDim.x % 8 == 0) {
    rank = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  }
  const int n_qb = p.hdr[H_NQB];
  DirectStage ds;                                  // large segments' K/V addressing, kept across segments
  ds.cur_b = -1;
  ds.cur_g = -1;
  ds.pbase = -(1 << 30);
  for (int vw = rank; vw < n_workers; vw += gridDim.x) {
    int a = wm.start(vw);
    const int b_end = min(a + wm.size(vw), U);
    if constexpr (HEADS) {                              // sequence Q-blocks: every wave writes its own rows
      heads_range<KIND, D, FAST>(pk, vw, wm, a, b_end);
      continue;
    }
    int q = find_qblock(p, 0, n_qb - 1, a, threadIdx.x & 63);
    while (a < b_end && q < n_qb) {
      const int S = p.unit_prefix[q], nq = p.unit_prefix[q + 1] - S;
      if (nq == 0) { ++q; continue; }
      const int u0 = a - S, u1 = min(b_end, S + nq) - S;
      const QBlock x = load_qblock(p, q);
      // (the large-only kernel runs every Q-block, the last few tokens of a
      // long sequence included, on the 128-row path)
      if (!LARGE && x.rows <= kSmallMaxRows && p.bm == nullptr) {
        // the maximal run of small Q-blocks from here, inside this worker's range
        int run_end = S + u1, qq = q + 1;
        while (run_end < b_end && qq < n_qb) {
          const int4 d = reinterpret_cast<const int4*>(p.qb_desc)[2 * qq];
          if (wave_uniform(d.w) * p.G > kSmallMaxRows) break;
          run_end = min(b_end, p.unit_prefix[qq + 1]);
          ++qq;
        }
        run_end = wave_uniform(run_end);
        small_range<KIND, D, FAST>(pk, vw, wm, a, run_end);
        a = run_end;
        while (q < n_qb && p.unit_prefix[q + 1] <= a) ++q;
        continue;
      }
      int t_lo = 0, t_hi = 0;
      qblock_tiles(p, x.ctx, x.pos_lo, x.pos_hi, t_lo, t_hi);
      const bool final_out = p.n_splits[q] == 1;
      const int slot = final_out ? 0 : p.slot_base[q] + (vw - wm.worker_of(S));
      if (!LARGE && x.rows <= kSmallMaxRows) small_segment<KIND, D, FAST>(pk, x, t_lo, t_hi, u0, u1, final_out, slot);
      else if constexpr (SMALL) {
        if (threadIdx.x == 0) p.hdr[H_ERROR] = E_QLEN_HINT;
        a = S + u1;
        ++q;
        continue;
      } else {
        large_segment<KIND, D, FAST, PATHS == kPathsLean>(pk, x, t_lo, t_hi, u0, u1, final_out, slot, ds);
      }
      if (!final_out && p.fused) finish_split<KIND, D>(p, q, x, p.n_splits[q], p.slot_base[q]);
      a = S + u1;
      ++q;
    }
  }
}

// The dynamic-LDS limit of a kernel build is raised once per device (the
// attribute is per device); the bit of a device is set only after the call
// succeeded, and concurrent first calls merely repeat the idempotent set.
template <int KIND, int D, bool FAST, int PATHS>
static hipError_t launch_attention_t(const KParams& p, int grid, hipStream_t stream) {
  const int lds = PATHS == kPathsLean ? Lds<KIND, D, FAST>::DYN_LEAN : Lds<KIND, D, FAST>::DYN;
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (!bit || !(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attention_kernel<KIND, D, FAST, PATHS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL((attention_kernel<KIND, D, FAST, PATHS>), dim3(grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <int KIND, int D, int PATHS>
static hipError_t launch_attention_kd(const KParams& p, int grid, hipStream_t stream) {
  return p.page_size >= kUnitKeys ? launch_attention_t<KIND, D, true, PATHS>(p, grid, stream)
                                  : launch_attention_t<KIND, D, false, PATHS>(p, grid, stream);
}

template <int PATHS>
static hipError_t launch_attention_s(const KParams& p, int kind, int grid, hipStream_t stream) {
  if (kind == KIND_F32) return p.D == 64 ? launch_attention_kd<KIND_F32, 64, PATHS>(p, grid, stream)
                                         : launch_attention_kd<KIND_F32, 128, PATHS>(p, grid, stream);
  if (kind == KIND_BF16) return p.D == 64 ? launch_attention_kd<KIND_BF16, 64, PATHS>(p, grid, stream)
                                          : launch_attention_kd<KIND_BF16, 128, PATHS>(p, grid, stream);
  return p.D == 64 ? launch_attention_kd<KIND_F8, 64, PATHS>(p, grid, stream)
                   : launch_attention_kd<KIND_F8, 128, PATHS>(p, grid, stream);
}

hipError_t launch_attention(const KParams& p, int kind, int grid, int paths, hipStream_t stream) {
  if (paths == kPathsHeads) return launch_attention_s<kPathsHeads>(p, kind, grid, stream);
  // the lean build: bf16 or fp8, d = 128, whole-tile pages, no block mask, a
  // landmark chunk of 0 or a multiple of 64, and K and V caches whose bytes
  // (any page, slot and dim of a head) lie within 2^31 of the head's base, so
  // that its DMAs address them with 32-bit offsets from one buffer resource
  const int64_t elt = kind == KIND_BF16 ? 2 : 1;
  auto span_ok = [&](int64_t sp, int64_t ss) {
    return sp > 0 && ss > 0 && (int64_t(p.num_pages) * sp + int64_t(kUnitKeys) * ss + p.D) * elt < (int64_t(1) << 31);
  };
  if (paths == kPathsLarge && kind != KIND_F32 && p.D == 128 && p.page_size >= kUnitKeys && p.bm == nullptr &&
      p.landmark % kUnitKeys == 0 && span_ok(p.k_sp, p.k_ss) && span_ok(p.v_sp, p.v_ss)) {
    return kind == KIND_BF16 ? launch_attention_t<KIND_BF16, 128, true, kPathsLean>(p, grid, stream)
                             : launch_attention_t<KIND_F8, 128, true, kPathsLean>(p, grid, stream);
  }
  if (paths == kPathsSmall) return launch_attention_s<kPathsSmall>(p, kind, grid, stream);
  if (paths == kPathsLarge) return launch_attention_s<kPathsLarge>(p, kind, grid, stream);
  return launch_attention_s<kPathsAll>(p, kind, grid, stream);
}

}  // namespace pa
