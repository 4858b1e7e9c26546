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

template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(KParams p) {
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  const float ninf = -__builtin_huge_valf();
  const int n_combine = p.hdr[H_NCOMBINE];
  constexpr int TPR = D / 8;
  for (int i = blockIdx.x; i < n_combine; i += gridDim.x) {
    const int q = p.combine_list[i];
    const QBlock x = load_qblock(p, q);
    const int ns = p.n_splits[q];
    const int sb = p.slot_base[q];
    for (int idx = threadIdx.x; idx < x.rows * TPR; idx += blockDim.x) {
      const int row = idx / TPR, d0 = (idx % TPR) * 8;
      float M = ninf;
      for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, p.part_lse[(sb + sp) * kLargeRows + row]);
      float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      float lse = ninf;
      if (M != ninf) {
        float z = 0.f;
        for (int sp = 0; sp < ns; ++sp) z += exp2f((p.part_lse[(sb + sp) * kLargeRows + row] - M) * kLog2e);
        lse = M + log2f(z) * kLn2;
        for (int sp = 0; sp < ns; ++sp) {
          const float ls = p.part_lse[(sb + sp) * kLargeRows + row];
          if (ls == ninf) continue;
          const float w = exp2f((ls - lse) * kLog2e);
          const float* src = p.part_o + ((int64_t)(sb + sp) * kLargeRows + row) * D + d0;
          const f32x4c a = *reinterpret_cast<const f32x4c*>(src);
          const f32x4c b = *reinterpret_cast<const f32x4c*>(src + 4);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            o[k] += w * a[k];
            o[4 + k] += w * b[k];
          }
        }
      }
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
