// Per-head projections around the absorbed decode (gfx950):
//   mla_absorb_q  q_lat[r, i, :] = q_nope[r, i, :] @ W_UK[i]   (K = 128, N = 512)
//   mla_up_v      o[r, i, :]     = o_lat[r, i, :]  @ W_UV[i]   (K = 512, N = 128)
// with r running over the b * s_q query tokens. The absorption trick
// ("DeepSeek-V3 Multi-head Latent Attention (MLA) 深度工程", section 2.4)
// moves W_UK onto the query so the decode scores against the latent, and
// since the decode output is linear in the latent rows, W_UV is applied once
// to the attention output instead of to every cached token (section 2.2).
//
// Each workgroup computes one head's 128-row x 64-column output tile with
// 32x32x16 bf16 MFMAs. The weight tile W[i][0:K][n0:n0+64] is staged in LDS
// once; its k runs down LDS rows, so the B operand (8 consecutive k of one
// column per lane) comes from transposed LDS reads. A rows stream from
// global memory straight into the A operand (16 contiguous bytes per lane).
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_host.h"

namespace mla {

constexpr int kGemmRows = 128;  // rows per workgroup: 4 waves x 32
constexpr int kGemmCols = 64;   // columns per workgroup: 2 MFMA tiles
constexpr int kGemmLdsStride = kGemmCols * 2 + 16;

template <int K, int N>
__global__ __launch_bounds__(256) void head_gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                        uint16_t* __restrict__ out, uint16_t* __restrict__ out_lo,
                                                        int R, int h) {
  __shared__ __attribute__((aligned(16))) char smem[K * kGemmLdsStride];
  MLA_LDS char* lds = (MLA_LDS char*)(smem);
  const int n0 = blockIdx.x * kGemmCols, r0 = blockIdx.y * kGemmRows, head = blockIdx.z;

  // stage W[head][:, n0 : n0 + 64] (row k of the tile = 128 contiguous bytes)
  const char* wsrc = reinterpret_cast<const char*>(W + (size_t)head * K * N + n0);
  constexpr int kChunks = K * kGemmCols / 8;
  for (int c = threadIdx.x; c < kChunks; c += 256) {
    const int k = c / (kGemmCols / 8), ch = c % (kGemmCols / 8);
    const u32x4 v = *reinterpret_cast<const u32x4*>(wsrc + (size_t)k * N * 2 + ch * 16);
    *(MLA_LDS u32x4*)(lds + k * kGemmLdsStride + ch * 16) = v;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, g = lane >> 5, j16 = lane & 15;
  const int row = r0 + wave * 32 + r32;
  const bool ok = row < R;
  const unsigned keep = ok ? 0xffffffffu : 0u;
  const u32x4* arow = reinterpret_cast<const u32x4*>(A + ((size_t)(ok ? row : 0) * h + head) * K) + g;
  // transposed-read address: k row 16 ks + 8 g + j16/4, column 16*((lane/16)&1) + 4*(j16&3)
  const int b_off = (8 * g + (j16 >> 2)) * kGemmLdsStride + (16 * ((lane >> 4) & 1) + 4 * (j16 & 3)) * 2;

  f32x16 c0 = f32x16{}, c1 = f32x16{};
#pragma unroll 4
  for (int ks = 0; ks < K / 16; ++ks) {
    const bf16x8 a = as_bf16x8(arow[2 * ks] & keep);
    const int o = b_off + 16 * ks * kGemmLdsStride;
    const bf16x8 b0 = cat4(lds_read_tr4(lds, o), lds_read_tr4(lds, o + 4 * kGemmLdsStride));
    const bf16x8 b1 = cat4(lds_read_tr4(lds, o + 64), lds_read_tr4(lds, o + 64 + 4 * kGemmLdsStride));
    c0 = mfma32(a, b0, c0);
    c1 = mfma32(a, b1, c1);
  }

  // lane holds C[row 8*(v/4) + 4*g + v%4][column l%32] of each tile
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int orow = r0 + wave * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
    if (orow < R) {
      const size_t o = ((size_t)orow * h + head) * N + n0 + r32;
      const __bf16 h0 = (__bf16)c0[v], h1 = (__bf16)c1[v];
      out[o] = __builtin_bit_cast(uint16_t, h0);
      out[o + 32] = __builtin_bit_cast(uint16_t, h1);
      if (out_lo) {
        out_lo[o] = bf16_bits(c0[v] - (float)h0);
        out_lo[o + 32] = bf16_bits(c1[v] - (float)h1);
      }
    }
  }
}

}  // namespace mla

using namespace mla;

static int check_ptr16(const char* fn, const void* p, const char* name) {
  if (!p) return set_error(MLA_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
  if (reinterpret_cast<uintptr_t>(p) % 16)
    return set_error(MLA_ERR_INVALID_ARG, "%s: %s must be 16-byte aligned", fn, name);
  return MLA_OK;
}

extern "C" int mla_absorb_q(const uint16_t* q_nope, const uint16_t* w_uk, uint16_t* q_lat, uint16_t* q_lat_lo,
                            int b, int s_q, int h, void* stream) {
  const char* fn = "mla_absorb_q";
  if (int rc = check_ptr16(fn, q_nope, "q_nope")) return rc;
  if (int rc = check_ptr16(fn, w_uk, "w_uk")) return rc;
  if (int rc = check_ptr16(fn, q_lat, "q_lat")) return rc;
  if (q_lat_lo && reinterpret_cast<uintptr_t>(q_lat_lo) % 16)
    return set_error(MLA_ERR_INVALID_ARG, "%s: q_lat_lo must be 16-byte aligned", fn);
  if (int rc = check_shape(fn, b, s_q, h)) return rc;
  const int R = b * s_q;
  dim3 grid(kDLat / kGemmCols, (R + kGemmRows - 1) / kGemmRows, h);
  hipLaunchKernelGGL((head_gemm_kernel<kDNope, kDLat>), grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                     q_nope, w_uk, q_lat, q_lat_lo, R, h);
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return clear_error();
}

extern "C" int mla_up_v(const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o, int b, int s_q, int h,
                        void* stream) {
  const char* fn = "mla_up_v";
  if (int rc = check_ptr16(fn, o_lat, "o_lat")) return rc;
  if (int rc = check_ptr16(fn, w_uv, "w_uv")) return rc;
  if (int rc = check_ptr16(fn, o, "o")) return rc;
  if (int rc = check_shape(fn, b, s_q, h)) return rc;
  const int R = b * s_q;
  dim3 grid(kDNope / kGemmCols, (R + kGemmRows - 1) / kGemmRows, h);
  hipLaunchKernelGGL((head_gemm_kernel<kDLat, kDNope>), grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                     o_lat, w_uv, o, static_cast<uint16_t*>(nullptr), R, h);
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return clear_error();
}
