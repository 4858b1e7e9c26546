// assign.hip — the Assign stage: one workgroup builds the task map.
//
// "Triton-TLE rewrite of Tencent HPC-Ops Attention", §1.2: Assign cuts every
// KV sequence into tiles and produces a load-balanced, GPU-resident task map
// for the persistent split-K workgroups; §3.3: the chunk length is chosen from
// the total load first, then each request is cut by its own KV length.  The
// map is integer-only and must equal the CPU specification bit for bit:
//   Q-blocks in (b, g) order, a large Q-block's token blocks zig-zag
//   (0, n-1, 1, n-2, ...); n_units = active 64-key tiles; prefix S;
//   L = force ? force : max(L_min, ceil(U / P)); worker w owns [wL, (w+1)L);
//   n_splits(q) = 0 | floor((S+n-1)/L) - floor(S/L) + 1; combine list = the
//   Q-blocks with n_splits != 1; slot_base = running sum over split Q-blocks.
#include "pa_device.h"

namespace pa {

constexpr int kAssignThreads = 1024;
constexpr int kAssignMaskLds = 64 * 1024;   // block masks up to this many bytes are staged in LDS

// Bytes of the block mask as a dense [B, H_m, n_q_tiles, n_k_tiles] array.
__host__ __device__ inline long long mask_elems(const KParams& p) {
  return p.bm == nullptr ? 0 : (long long)p.B * p.bm_heads * p.bm_nq * p.bm_nk;
}

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

__global__ __launch_bounds__(kAssignThreads) void assign_kernel(KParams p) {
  __shared__ int sh[kAssignThreads / 64 + 1];
  __shared__ int err;
  extern __shared__ uint8_t mask_lds[];
  const int tid = threadIdx.x;
  if (tid == 0) err = E_NONE;
  // A small block mask is copied into LDS first (independent byte loads from
  // every thread) so that the per-Q-block tile counts below read LDS instead of
  // issuing one dependent global load per tile.
  const long long melems = mask_elems(p);
  const bool staged = melems > 0 && melems <= kAssignMaskLds;
  if (staged) {
    for (int i = tid; i < (int)melems; i += kAssignThreads) {
      int r = i;
      const int kt = r % p.bm_nk; r /= p.bm_nk;
      const int qt = r % p.bm_nq; r /= p.bm_nq;
      const int hm = r % p.bm_heads;
      const int b = r / p.bm_heads;
      mask_lds[i] = p.bm[b * p.bm_sb + hm * p.bm_sh + qt * p.bm_sq + kt * p.bm_sk] != 0;
    }
  }
  __syncthreads();

  // 0. metadata checks: qsl is a non-decreasing prefix ending at total_q, q_len <= seq_len
  for (int b = tid; b < p.B; b += kAssignThreads) {
    const int a = p.qsl[b], c = p.qsl[b + 1];
    if ((b == 0 && a != 0) || c < a || (b == p.B - 1 && c != p.total_q)) atomicMax(&err, (int)E_QSL);
    else if (c - a > p.seq_lens[b]) atomicMax(&err, (int)E_QLEN);
  }
  __syncthreads();
  if (err != E_NONE) {
    if (tid == 0) {
      for (int i = 0; i < kHeaderInts; ++i) p.hdr[i] = 0;
      p.hdr[H_P] = p.P;
      p.hdr[H_ERROR] = err;
      p.hdr[H_MAXSLOTS] = p.max_slots;
    }
    return;
  }

  // 1. Q-blocks per sequence -> first Q-block index of each sequence
  const int nt_large = kLargeRows / p.G;
  int carry = 0, tot;
  for (int c0 = 0; c0 < p.B; c0 += kAssignThreads) {
    const int b = c0 + tid;
    int nqb = 0;
    if (b < p.B) {
      const int ql = p.qsl[b + 1] - p.qsl[b];
      nqb = ql <= 0 ? 0 : (ql * p.G <= kSmallMaxRows ? 1 : (ql + nt_large - 1) / nt_large);
      nqb *= p.Hkv;
    }
    const int ex = block_exclusive_scan(nqb, &tot, sh);
    if (b < p.B) p.seq_qb_base[b] = carry + ex;
    carry += tot;
  }
  if (tid == 0) p.seq_qb_base[p.B] = carry;
  const int n_qb = carry;
  __syncthreads();

  // 2. descriptors and unit counts (counts parked in unit_prefix[q + 1])
  for (int q = tid; q < n_qb; q += kAssignThreads) {
    int lo = 0, hi = p.B - 1;                      // last b with base[b] <= q
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.seq_qb_base[mid] <= q) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int per_g = (p.seq_qb_base[b + 1] - p.seq_qb_base[b]) / p.Hkv;
    const int rem = q - p.seq_qb_base[b];
    const int g = rem / per_g, t = rem % per_g;
    const int q0 = p.qsl[b], ql = p.qsl[b + 1] - q0, ctx = p.seq_lens[b];
    const int ntl = ql * p.G <= kSmallMaxRows ? ql : nt_large;
    // zig-zag over the token blocks (spreads short and long Q-blocks evenly)
    const int zi = (t & 1) ? per_g - 1 - (t >> 1) : (t >> 1);
    const int t0 = zi * ntl;
    const int nt = min(ntl, ql - t0);
    reinterpret_cast<int4*>(p.qb_desc)[2 * q] = make_int4(b, g, t0, nt);
    reinterpret_cast<int4*>(p.qb_desc)[2 * q + 1] = make_int4(q0, ql, ctx, 0);   // saves the kernel two dependent loads
    const int pos_lo = ctx - ql + t0, pos_hi = pos_lo + nt - 1;
    int t_lo, t_hi, n = 0;
    if (qblock_tiles(p, ctx, pos_lo, pos_hi, t_lo, t_hi)) {
      if (p.bm == nullptr) {
        n = t_hi - t_lo + 1;
      } else {
        // walk the mask columns kt (T = block_mask_tile keys = upt 64-key
        // tiles): a set column adds its tiles that lie in [t_lo, t_hi]
        const int upt = p.bm_tile / kUnitKeys;
        const int kt_lo = t_lo / upt, kt_hi = min(t_hi / upt, p.bm_nk - 1);
        const int qt0 = pos_lo / p.bm_tile, qt1 = min(pos_hi / p.bm_tile, p.bm_nq - 1);
        const int h0 = p.bm_heads == 1 ? 0 : g * p.G, h1 = p.bm_heads == 1 ? 1 : (g + 1) * p.G;
        for (int kt = kt_lo; kt <= kt_hi; ++kt) {
          bool on = false;
          for (int hm = h0; hm < h1 && !on; ++hm)
            for (int qt = qt0; qt <= qt1 && !on; ++qt)
              on = staged ? mask_lds[(((long long)b * p.bm_heads + hm) * p.bm_nq + qt) * p.bm_nk + kt] != 0
                          : p.bm[b * p.bm_sb + hm * p.bm_sh + qt * p.bm_sq + kt * p.bm_sk] != 0;
          if (on) n += min(t_hi, kt * upt + upt - 1) - max(t_lo, kt * upt) + 1;
        }
      }
    }
    p.unit_prefix[q + 1] = n;
  }
  __syncthreads();

  // 3. unit prefix
  carry = 0;
  for (int c0 = 0; c0 < n_qb; c0 += kAssignThreads) {
    const int q = c0 + tid;
    const int n = q < n_qb ? p.unit_prefix[q + 1] : 0;
    const int ex = block_exclusive_scan(n, &tot, sh);
    if (q < n_qb) p.unit_prefix[q + 1] = carry + ex + n;
    carry += tot;
  }
  if (tid == 0) p.unit_prefix[0] = 0;
  const int U = carry;
  const int L = p.force_L > 0 ? p.force_L : max(p.L_min, (U + p.P - 1) / p.P);
  __syncthreads();

  // 4. splits, combine list, partial slots
  int c_carry = 0, s_carry = 0, ctot, stot;
  for (int c0 = 0; c0 < n_qb; c0 += kAssignThreads) {
    const int q = c0 + tid;
    int ns = 1;
    if (q < n_qb) {
      const int S = p.unit_prefix[q], n = p.unit_prefix[q + 1] - S;
      ns = n == 0 ? 0 : (S + n - 1) / L - S / L + 1;
      p.n_splits[q] = ns;
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
    p.hdr[H_NWORKERS] = over ? 0 : (U ? (U + L - 1) / L : 0);
    p.hdr[H_ERROR] = over ? E_SLOTS : E_NONE;
    p.hdr[H_MAXSLOTS] = p.max_slots;
    for (int i = H_MAXSLOTS + 1; i < kHeaderInts; ++i) p.hdr[i] = 0;
  }
}

hipError_t launch_assign(const KParams& p, hipStream_t stream) {
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&assign_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kAssignMaskLds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const long long me = mask_elems(p);
  const int lds = (me > 0 && me <= kAssignMaskLds) ? (int)((me + 15) & ~15LL) : 0;
  hipLaunchKernelGGL(assign_kernel, dim3(1), dim3(kAssignThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace pa
