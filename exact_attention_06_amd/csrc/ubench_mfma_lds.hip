// ubench_mfma_lds.hip - measurement only (not part of libfa.so): how LDS fragment reads
// interleaved with v_mfma_f32_32x32x16_bf16 change the rate at which the matrix cores issue.
//
// Every workgroup is 8 waves (two per SIMD, as in the attention kernels), one per CU. Per loop
// iteration a wave issues NM independent MFMAs whose A operands come from LDS reads issued in
// the previous iteration (the kernels' prefetch pattern), waiting for them at the iteration's
// end. The reads use the hd256 forward kernel's own fragment layouts: K rows padded to 528 B
// read 16 bytes per lane (ds_read_b128), V rows padded to 576 B read through the transpose
// read (two ds_read_b64_tr_b16 per fragment). Modes:
//   0: 2 MFMAs, no LDS reads
//   1: 2 MFMAs + 2 K fragments  (1 KB of LDS reads per MFMA, as in S^T = K Q^T)
//   2: 2 MFMAs + 2 V fragments  (1 KB per MFMA through the transpose read, as in O^T += V^T P^T)
//   3: 4 MFMAs + 2 K fragments  (0.5 KB per MFMA: each fragment feeds two MFMAs)
//   4: 4 MFMAs + 2 V fragments  (0.5 KB per MFMA)
// All LDS offsets stay below 20 KB of the 64 KB array.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int MODE>
__global__ void __launch_bounds__(512, 1) ub_kernel(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[65536];
  const int lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  for (int i = threadIdx.x; i < 65536 / 16; i += 512) ((u32x4*)buf)[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  constexpr int KROW = 528, VROW = 576;
  const int k_rd = l32 * KROW + hh * 16;
  const int grp = lane >> 4, gi = lane & 15;
  const int v_rd = (4 * (grp >> 1) + (gi >> 2)) * VROW + (2 * (grp & 1) + ((gi & 3) >> 1)) * 16 + (gi & 1) * 8;
  auto kread = [&](int t) -> u32x4 { return *(const u32x4*)(buf + k_rd + (t & 15) * 32); };
  auto vread = [&](int i) -> u32x4 {
    const int u = (i >> 3) & 1, md = i & 7;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + v_rd + 16 * u * VROW + md * 64));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + v_rd + (16 * u + 8) * VROW + md * 64));
    u32x4 r;
    r[0] = __builtin_bit_cast(u32x2, lo)[0];
    r[1] = __builtin_bit_cast(u32x2, lo)[1];
    r[2] = __builtin_bit_cast(u32x2, hi)[0];
    r[3] = __builtin_bit_cast(u32x2, hi)[1];
    return r;
  };
  bf16x8 y;
  for (int e = 0; e < 8; ++e) y[e] = (__bf16)0.5f;
  f32x16 a0 = {}, a1 = {}, a2 = {}, a3 = {};
  u32x4 f0 = {}, f1 = {};
  for (int it = 0; it < iters; ++it) {
    const int j = (it * 2) & 15;
    if constexpr (MODE == 0) {
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f0), y, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f1), y, a1, 0, 0, 0);
    } else {
      const u32x4 n0 = (MODE == 1 || MODE == 3) ? kread(j) : vread(j);
      const u32x4 n1 = (MODE == 1 || MODE == 3) ? kread(j + 1) : vread(j + 1);
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f0), y, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f1), y, a1, 0, 0, 0);
      if constexpr (MODE == 3 || MODE == 4) {
        a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f0), __builtin_bit_cast(bf16x8, f1),
                                                     a2, 0, 0, 0);
        a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f1), __builtin_bit_cast(bf16x8, f0),
                                                     a3, 0, 0, 0);
      }
      f0 = n0;
      f1 = n1;
    }
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += a0[i] + a1[i] + a2[i] + a3[i];
  s += (float)(f0[0] ^ f1[1]);
  out[blockIdx.x * 512 + threadIdx.x] = s;
}

extern "C" int ub_mfmas_per_iter(int mode) { return mode >= 3 ? 4 : 2; }

extern "C" int ub_run(int mode, float* out, int iters, int blocks, void* stream) {
  if (blocks <= 0 || iters <= 0) return -3;
  hipStream_t st = (hipStream_t)stream;
  switch (mode) {
    case 0: hipLaunchKernelGGL(ub_kernel<0>, dim3(blocks), dim3(512), 0, st, out, iters); break;
    case 1: hipLaunchKernelGGL(ub_kernel<1>, dim3(blocks), dim3(512), 0, st, out, iters); break;
    case 2: hipLaunchKernelGGL(ub_kernel<2>, dim3(blocks), dim3(512), 0, st, out, iters); break;
    case 3: hipLaunchKernelGGL(ub_kernel<3>, dim3(blocks), dim3(512), 0, st, out, iters); break;
    case 4: hipLaunchKernelGGL(ub_kernel<4>, dim3(blocks), dim3(512), 0, st, out, iters); break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
