// combine.hip — the Combine stage: LSE-weighted merge of split partials.
//
// "Triton-TLE rewrite of Tencent HPC-Ops Attention", §1.2: Combine
// re-normalises the partial outputs of the KV chunks by their LSE, which is
// mathematically the same as full attention; §3.3 gives the same merge on raw
// online-softmax states.  For every row of a split Q-block:
//   M = max_s LSE_s;  LSE = M + ln sum_s exp(LSE_s - M);  O = sum_s exp(LSE_s - LSE) O_s.
// Parts with LSE_s = -inf weigh 0; a row whose parts are all -inf (or a
// Q-block with no unit at all) gets O = 0 and LSE = -inf.
#include "pa_device.h"

namespace pa {

typedef float f32x4c __attribute__((ext_vector_type(4)));
typedef unsigned u32x4c __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned pack_bf16x2_c(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

// One split merged into a running (m, z, o) state (natural-log domain LSEs):
// m = running max, z = sum of e^(LSE_s - m), o = sum of e^(LSE_s - m) O_s.
struct MergeState {
  float m, z, o[8];
};

__device__ __forceinline__ void merge_part(MergeState& st, float ls, const float* src) {
  constexpr float kLog2e = 1.4426950408889634f;
  if (!(ls > -__builtin_huge_valf())) return;          // an empty part weighs nothing
  const f32x4c a = *reinterpret_cast<const f32x4c*>(src);
  const f32x4c b = *reinterpret_cast<const f32x4c*>(src + 4);
  const float m_new = fmaxf(st.m, ls);
  const float alpha = st.m == -__builtin_huge_valf() ? 0.f : exp2f((st.m - m_new) * kLog2e);
  const float w = exp2f((ls - m_new) * kLog2e);
  st.z = st.z * alpha + w;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    st.o[k] = st.o[k] * alpha + w * a[k];
    st.o[4 + k] = st.o[4 + k] * alpha + w * b[k];
  }
  st.m = m_new;
}

__device__ __forceinline__ void merge_state(MergeState& st, const MergeState& other) {
  constexpr float kLog2e = 1.4426950408889634f;
  if (other.m == -__builtin_huge_valf()) return;
  const float m_new = fmaxf(st.m, other.m);
  const float a = st.m == -__builtin_huge_valf() ? 0.f : exp2f((st.m - m_new) * kLog2e);
  const float b = exp2f((other.m - m_new) * kLog2e);
  st.z = st.z * a + other.z * b;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = st.o[k] * a + other.o[k] * b;
  st.m = m_new;
}

// A workgroup per split Q-block.  Thread (group, row, 8 dims): when a
// Q-block's rows need fewer than 256 threads, the spare threads form groups
// that take every groups-th split, and the groups' states are merged through
// LDS, so that a Q-block cut into many splits (a long decode) is read with
// many loads in flight instead of one chain per row.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(KParams p) {
  constexpr float kLn2 = 0.6931471805599453f;
  const float ninf = -__builtin_huge_valf();
  __shared__ MergeState red[256];
  const bool stat = p.static_S > 0;
  // static split: every Q-block is a candidate, its split count recomputed
  const int n_combine = stat ? p.B * p.Hkv : p.hdr[H_NCOMBINE];
  constexpr int TPR = D / 8;
  for (int i = blockIdx.x; i < n_combine; i += gridDim.x) {
    int q, ns, sb;
    QBlock x;
    if (stat) {
      q = i;
      if (static_qblock(p, q, x) != E_NONE) continue;
      ns = static_split(p, x).ns;
      if (ns < 2) continue;                          // written by the attention kernel
      sb = q * p.static_S;
    } else {
      q = p.combine_list[i];
      x = load_qblock(p, q);
      ns = p.n_splits[q];
      sb = p.slot_base[q];
    }
    const int per = x.rows * TPR;                      // threads one pass over the rows needs
    const int groups = per >= 256 ? 1 : 256 / per;
    for (int base = 0; base < per; base += 256) {
      const int t = threadIdx.x;
      const int grp = groups > 1 ? t / per : 0;
      const int idx = groups > 1 ? t % per : base + t;
      const bool live = grp < groups && idx < per;
      const int row = idx / TPR, d0 = (idx % TPR) * 8;
      MergeState st;
      st.m = ninf;
      st.z = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) st.o[k] = 0.f;
      if (live) {
        for (int sp = grp; sp < ns; sp += groups) {
          const float ls = p.part_lse[(sb + sp) * kLargeRows + row];
          merge_part(st, ls, p.part_o + ((int64_t)(sb + sp) * kLargeRows + row) * D + d0);
        }
      }
      if (groups > 1) {
        red[t] = st;
        __syncthreads();
        if (live && grp == 0)
          for (int gq = 1; gq < groups; ++gq) merge_state(st, red[gq * per + idx]);
        __syncthreads();
      }
      if (live && grp == 0) {
        const bool empty = !(st.z > 0.f);
        const float inv = empty ? 0.f : 1.f / st.z;
        const float lse = empty ? ninf : st.m + logf(st.z);
        float o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = st.o[k] * inv;
        const int tok = x.q0 + x.t0 + row / p.G, head = x.g * p.G + row % p.G;
        if constexpr (OUT_F32) {
          float* dst = reinterpret_cast<float*>(p.out) + tok * p.o_st + head * p.o_sh + d0;
          *reinterpret_cast<f32x4c*>(dst) = f32x4c{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<f32x4c*>(dst + 4) = f32x4c{o[4], o[5], o[6], o[7]};
        } else {
          char* dst = reinterpret_cast<char*>(p.out) + (tok * p.o_st + head * p.o_sh + d0) * 2;
          *reinterpret_cast<u32x4c*>(dst) = u32x4c{pack_bf16x2_c(o[0], o[1]), pack_bf16x2_c(o[2], o[3]),
                                                   pack_bf16x2_c(o[4], o[5]), pack_bf16x2_c(o[6], o[7])};
        }
        if (d0 == 0) p.lse[tok * p.l_st + head * p.l_sh] = lse;
      }
    }
  }
}

hipError_t launch_combine(const KParams& p, bool out_f32, int grid, hipStream_t stream) {
  if (p.D == 64) {
    if (out_f32) hipLaunchKernelGGL((combine_kernel<64, true>), dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((combine_kernel<64, false>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    if (out_f32) hipLaunchKernelGGL((combine_kernel<128, true>), dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((combine_kernel<128, false>), dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
