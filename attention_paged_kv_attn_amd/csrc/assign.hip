// assign.hip — the Assign stage: one workgroup builds the task map (with a
// block mask, a grid counts the units between its two halves).
//
// "Triton-TLE rewrite of Tencent HPC-Ops Attention", §1.2: Assign cuts every
// KV sequence into tiles and produces a load-balanced, GPU-resident task map
// for the persistent split-K workgroups; §3.3: the chunk length is chosen from
// the total load first, then each request is cut by its own KV length.  The
// map is integer-only and must equal the CPU specification bit for bit:
//   Q-blocks in (b, g) order, a large Q-block's token blocks zig-zag
//   (0, n-1, 1, n-2, ...); n_units = active 64-key tiles; prefix S;
//   (or one Q-block per sequence, units = its (tile, kv head) pairs, kv head
//   fastest); L = force ? force : max(L_min, ceil(U / P)); worker pair k owns
//   [2kL, 2kL + 2L), the first L0 units to worker 2k (L0 from the pair
//   weight, L0 = L at 50); worker_of(u) as in WorkerMap;
//   n_splits(q) = 0 | worker_of(S+n-1) - worker_of(S) + 1; combine list = the
//   Q-blocks with n_splits != 1; slot_base = running sum over split Q-blocks.
#include <algorithm>

#include "pa_device.h"

namespace pa {

constexpr int kAssignThreads = 1024;

// Exclusive prefix sum over the workgroup; *total gets the sum.  `sh` holds
// kAssignThreads / 64 + 1 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kAssignThreads / 64 ? sh[lane] : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(w, d);
      if (lane >= d) w += y;
    }
    if (lane < kAssignThreads / 64) sh[lane] = w;      // inclusive wave totals
    if (lane == kAssignThreads / 64 - 1) sh[kAssignThreads / 64] = w;
  }
  __syncthreads();
  const int base = wave ? sh[wave - 1] : 0;
  *total = sh[kAssignThreads / 64];
  __syncthreads();
  return base + x - v;
}

// Steps 0 and 1 (one workgroup): metadata checks, then the first Q-block of
// every sequence.  Returns n_qb, or -1 after writing an error header.
// The single-workgroup path keeps the per-sequence bases and the per-Q-block
// counts in LDS when they fit, so that the binary searches and the prefix pass
// read LDS instead of a chain of global loads.
constexpr int kSeqLds = 2048;      // sequences + 1
constexpr int kQbLds = 8192;       // Q-blocks + 1

__device__ int assign_sequences(const KParams& p, int* sh, int* err, int* base_lds) {
  const int tid = threadIdx.x;
  if (tid == 0) *err = E_NONE;
  __syncthreads();
  // 0. metadata checks: qsl is a non-decreasing prefix ending at total_q, q_len <= seq_len
  for (int b = tid; b < p.B; b += kAssignThreads) {
    const int a = p.qsl[b], c = p.qsl[b + 1];
    if ((b == 0 && a != 0) || c < a || (b == p.B - 1 && c != p.total_q)) atomicMax(err, (int)E_QSL);
    else if (c - a > p.seq_lens[b]) atomicMax(err, (int)E_QLEN);
    else if ((p.max_q_len > 0 && c - a > p.max_q_len) || (c > a && c - a < p.min_q_len))
      atomicMax(err, (int)E_QLEN_HINT);
  }
  __syncthreads();
  if (*err != E_NONE) {
    if (tid == 0) {
      for (int i = 0; i < kHeaderInts; ++i) p.hdr[i] = 0;
      p.hdr[H_P] = p.P;
      p.hdr[H_ERROR] = *err;
      p.hdr[H_MAXSLOTS] = p.max_slots;
    }
    return -1;
  }
  // 1. Q-blocks per sequence -> first Q-block index of each sequence
  const int nt_large = kLargeRows / p.G;
  int carry = 0, tot;
  for (int c0 = 0; c0 < p.B; c0 += kAssignThreads) {
    const int b = c0 + tid;
    int nqb = 0;
    if (b < p.B) {
      const int ql = p.qsl[b + 1] - p.qsl[b];
      if (p.seq_qb) {
        nqb = ql > 0 ? 1 : 0;                       // one Q-block with every query head
      } else {
        nqb = ql <= 0 ? 0 : (ql * p.G <= kSmallMaxRows ? 1 : (ql + nt_large - 1) / nt_large);
        nqb *= p.Hkv;
      }
    }
    const int ex = block_exclusive_scan(nqb, &tot, sh);
    if (b < p.B) {
      p.seq_qb_base[b] = carry + ex;
      if (base_lds) base_lds[b] = carry + ex;
    }
    carry += tot;
  }
  if (tid == 0) {
    p.seq_qb_base[p.B] = carry;
    if (base_lds) base_lds[p.B] = carry;
  }
  __syncthreads();
  return carry;
}

// Step 2 for one Q-block: its descriptor (written) and its tile range.
struct QbTiles {
  int b, g, pos_lo, pos_hi, t_lo, t_hi;
  bool any;
};
// `base`: the per-sequence first Q-block (LDS copy or the workspace array)
__device__ __forceinline__ QbTiles assign_descriptor(const KParams& p, int q, const int* base) {
  int lo = 0, hi = p.B - 1;                        // last b with base[b] <= q
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= q) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int q0 = p.qsl[b], ql = p.qsl[b + 1] - q0, ctx = p.seq_lens[b];
  int g = 0, t0 = 0, nt = ql;                        // a sequence Q-block: every head, every token
  if (!p.seq_qb) {
    const int nt_large = kLargeRows / p.G;
    const int per_g = (base[b + 1] - base[b]) / p.Hkv;
    const int rem = q - base[b];
    g = rem / per_g;
    const int t = rem % per_g;
    const int ntl = ql * p.G <= kSmallMaxRows ? ql : nt_large;
    // zig-zag over the token blocks (spreads short and long Q-blocks evenly)
    const int zi = (t & 1) ? per_g - 1 - (t >> 1) : (t >> 1);
    t0 = zi * ntl;
    nt = min(ntl, ql - t0);
  }
  reinterpret_cast<int4*>(p.qb_desc)[2 * q] = make_int4(b, g, t0, nt);
  reinterpret_cast<int4*>(p.qb_desc)[2 * q + 1] = make_int4(q0, ql, ctx, 0);   // saves the kernel two dependent loads
  QbTiles r;
  r.b = b;
  r.g = g;
  r.pos_lo = ctx - ql + t0;
  r.pos_hi = r.pos_lo + nt - 1;
  r.any = qblock_tiles(p, ctx, r.pos_lo, r.pos_hi, r.t_lo, r.t_hi);
  return r;
}

// Steps 3 and 4 (one workgroup): unit prefix, L, splits, combine list, slots, header.
// `pre`: LDS copy of unit_prefix (counts parked at [q + 1] on entry), or null
// to work on the workspace array
__device__ void assign_splits(const KParams& p, int n_qb, int* sh, int* pre) {
  const int tid = threadIdx.x;
  int* up = pre ? pre : p.unit_prefix;
  // 3. unit prefix
  int carry = 0, tot;
  for (int c0 = 0; c0 < n_qb; c0 += kAssignThreads) {
    const int q = c0 + tid;
    const int n = q < n_qb ? up[q + 1] : 0;
    const int ex = block_exclusive_scan(n, &tot, sh);
    if (q < n_qb) {
      up[q + 1] = carry + ex + n;
      if (pre) p.unit_prefix[q + 1] = carry + ex + n;
    }
    carry += tot;
  }
  if (tid == 0) {
    p.unit_prefix[0] = 0;
    if (pre) pre[0] = 0;
  }
  const int U = carry;
  const int L = p.force_L > 0 ? p.force_L : max(p.L_min, (U + p.P - 1) / p.P);
  const WorkerMap wm{L, WorkerMap::first_len(L, p.pair_w)};
  __syncthreads();

  // 4. splits, combine list, partial slots
  int c_carry = 0, s_carry = 0, ctot, stot;
  for (int c0 = 0; c0 < n_qb; c0 += kAssignThreads) {
    const int q = c0 + tid;
    int ns = 1;
    if (q < n_qb) {
      const int S = up[q], n = up[q + 1] - S;
      ns = n == 0 ? 0 : wm.worker_of(S + n - 1) - wm.worker_of(S) + 1;
      p.n_splits[q] = ns;
      p.done[q] = 0;
    }
    const int in_c = (q < n_qb && ns != 1) ? 1 : 0;
    const int in_s = (q < n_qb && ns >= 2) ? ns : 0;
    const int cx = block_exclusive_scan(in_c, &ctot, sh);
    const int sx = block_exclusive_scan(in_s, &stot, sh);
    if (q < n_qb) {
      if (in_c) p.combine_list[c_carry + cx] = q;
      p.slot_base[q] = in_s ? s_carry + sx : -1;
    }
    c_carry += ctot;
    s_carry += stot;
  }
  if (tid == 0) {
    const bool over = s_carry > p.max_slots;
    p.hdr[H_U] = over ? 0 : U;
    p.hdr[H_P] = p.P;
    p.hdr[H_L] = L;
    p.hdr[H_NQB] = n_qb;
    p.hdr[H_NSLOTS] = s_carry;
    p.hdr[H_NCOMBINE] = over ? 0 : c_carry;
    p.hdr[H_NWORKERS] = over ? 0 : (U ? wm.worker_of(U - 1) + 1 : 0);
    p.hdr[H_ERROR] = over ? E_SLOTS : E_NONE;
    p.hdr[H_MAXSLOTS] = p.max_slots;
    p.hdr[H_L0] = wm.L0;
    for (int i = H_L0 + 1; i < kHeaderInts; ++i) p.hdr[i] = 0;
  }
}

// Without a block mask: one workgroup does every step (unit counts are closed forms).
__global__ __launch_bounds__(kAssignThreads) void assign_kernel(KParams p) {
  __shared__ int sh[kAssignThreads / 64 + 1];
  __shared__ int err;
  __shared__ int base_lds[kSeqLds];
  __shared__ int pre_lds[kQbLds];
  int* bl = p.B + 1 <= kSeqLds ? base_lds : nullptr;
  const int n_qb = assign_sequences(p, sh, &err, bl);
  if (n_qb < 0) return;
  int* pl = n_qb + 1 <= kQbLds ? pre_lds : nullptr;
  // 2. descriptors and unit counts (counts parked at [q + 1])
  for (int q = threadIdx.x; q < n_qb; q += kAssignThreads) {
    const QbTiles r = assign_descriptor(p, q, bl ? bl : p.seq_qb_base);
    // a sequence Q-block's units are its (tile, kv head) pairs
    const int n = r.any ? (r.t_hi - r.t_lo + 1) * (p.seq_qb ? p.Hkv : 1) : 0;
    if (pl) pl[q + 1] = n;
    else p.unit_prefix[q + 1] = n;
  }
  __syncthreads();
  assign_splits(p, n_qb, sh, pl);
}

// With a block mask the unit counts are the expensive part, so they get a
// grid of their own between the two single-workgroup halves: one wave per
// Q-block, its lanes over the mask columns (independent loads, summed by a
// wave reduction).  The halves pass their state through the workspace: the
// first leaves n_qb in seq_qb_base[B] and E_NONE in the error word.
__global__ __launch_bounds__(kAssignThreads) void assign_begin_kernel(KParams p) {
  __shared__ int sh[kAssignThreads / 64 + 1];
  __shared__ int err;
  const int n_qb = assign_sequences(p, sh, &err, nullptr);
  if (n_qb >= 0 && threadIdx.x == 0) p.hdr[H_ERROR] = E_NONE;
}

constexpr int kCountThreads = 256;

__global__ __launch_bounds__(kCountThreads) void assign_count_kernel(KParams p) {
  if (p.hdr[H_ERROR] != E_NONE) return;
  const int n_qb = p.seq_qb_base[p.B];
  const int lane = threadIdx.x & 63;
  const int waves = kCountThreads / 64;
  const int upt = p.bm_tile / kUnitKeys;
  for (int q = blockIdx.x * waves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); q < n_qb; q += gridDim.x * waves) {
    QbTiles r;
    if (lane == 0) r = assign_descriptor(p, q, p.seq_qb_base);
    r.b = __shfl(r.b, 0);
    r.g = __shfl(r.g, 0);
    r.pos_lo = __shfl(r.pos_lo, 0);
    r.pos_hi = __shfl(r.pos_hi, 0);
    r.t_lo = __shfl(r.t_lo, 0);
    r.t_hi = __shfl(r.t_hi, 0);
    r.any = __shfl((int)r.any, 0) != 0;
    int cnt = 0;
    if (r.any) {
      // a mask column kt (block_mask_tile keys = upt 64-key tiles) that is set
      // for some head and query tile of the Q-block adds its tiles in [t_lo, t_hi]
      const int kt_lo = r.t_lo / upt, kt_hi = min(r.t_hi / upt, p.bm_nk - 1);
      const int qt0 = r.pos_lo / p.bm_tile, qt1 = min(r.pos_hi / p.bm_tile, p.bm_nq - 1);
      const int h0 = p.bm_heads == 1 ? 0 : r.g * p.G, h1 = p.bm_heads == 1 ? 1 : (r.g + 1) * p.G;
      const uint8_t* base = p.bm + r.b * p.bm_sb;
      for (int kt = kt_lo + lane; kt <= kt_hi; kt += 64) {
        bool on = false;
        for (int hm = h0; hm < h1; ++hm)
          for (int qt = qt0; qt <= qt1; ++qt) on |= base[hm * p.bm_sh + qt * p.bm_sq + kt * p.bm_sk] != 0;
        if (on) cnt += min(r.t_hi, kt * upt + upt - 1) - max(r.t_lo, kt * upt) + 1;
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) cnt += __shfl_xor(cnt, d);
    if (lane == 0) p.unit_prefix[q + 1] = cnt;
  }
}

__global__ __launch_bounds__(kAssignThreads) void assign_end_kernel(KParams p) {
  __shared__ int sh[kAssignThreads / 64 + 1];
  if (p.hdr[H_ERROR] != E_NONE) return;
  assign_splits(p, p.seq_qb_base[p.B], sh, nullptr);
}

// Static split: no task map, only the header (error word cleared, sizes for
// inspection) written before the attention kernel.
__global__ __launch_bounds__(256) void static_begin_kernel(KParams p) {
  for (int q = threadIdx.x; q < p.B * p.Hkv; q += blockDim.x) p.done[q] = 0;
  if (threadIdx.x == 0) {
    const int n_qb = p.B * p.Hkv;
    p.hdr[H_U] = 0;
    p.hdr[H_P] = p.P;
    p.hdr[H_L] = 0;
    p.hdr[H_NQB] = n_qb;
    p.hdr[H_NSLOTS] = p.static_S > 1 ? n_qb * p.static_S : 0;
    p.hdr[H_NCOMBINE] = p.static_S > 1 ? n_qb : 0;
    p.hdr[H_NWORKERS] = n_qb * p.static_S;
    p.hdr[H_ERROR] = E_NONE;
    p.hdr[H_MAXSLOTS] = p.max_slots;
  }
}

hipError_t launch_static_begin(const KParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(static_begin_kernel, dim3(1), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_assign(const KParams& p, hipStream_t stream) {
  if (p.bm == nullptr) {
    hipLaunchKernelGGL(assign_kernel, dim3(1), dim3(kAssignThreads), 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(assign_begin_kernel, dim3(1), dim3(kAssignThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = kCountThreads / 64;
  const int grid = (int)std::min<long long>(4096, ((long long)p.n_qb_max + waves - 1) / waves);
  hipLaunchKernelGGL(assign_count_kernel, dim3(grid > 0 ? grid : 1), dim3(kCountThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(assign_end_kernel, dim3(1), dim3(kAssignThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
