// Per-head projections around the absorbed decode (gfx950):
//   mla_absorb_q  q_lat[r, i, :] = q_nope[r, i, :] @ W_UK[i]   (K = 128, N = 512)
//   mla_up_v      o[r, i, :]     = o_lat[r, i, :]  @ W_UV[i]   (K = 512, N = 128)
// with r running over the b * s_q query tokens. The absorption trick
// ("DeepSeek-V3 Multi-head Latent Attention (MLA) 深度工程", section 2.4)
// moves W_UK onto the query so the decode scores against the latent, and
// since the decode output is linear in the latent rows, W_UV is applied once
// to the attention output instead of to every cached token (section 2.2).
//
// Each workgroup computes one head's 128-row x NT-column output tile (four
// waves of 32 rows). The tiles of one head are consecutive workgroups on one
// XCD (workgroup ids go round-robin over the 8 XCDs), so the A rows and the
// weight columns that several tiles of the head read come from that XCD's L2
// after the first read. The tile is computed with 32x32x16 bf16 MFMAs, as the
// transposed product
// C^T = W^T A^T. The weight tile W[i][0:K][n0:n0+NT] is staged in LDS once
// and read back transposed as the A operand; each lane's B operand (8
// consecutive k of one row of A) is 16 contiguous bytes of that row, loaded
// straight from HBM. In the C^T layout a lane holds 4 consecutive output
// columns of one row per element group, so the tile goes to LDS with 8-byte
// writes and leaves as whole row segments (NT * 2 contiguous bytes per row).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mla_device.h"
#include "mla_host.h"
#include "mla_plan.h"

namespace mla {

constexpr int kGemmRows = 128;  // rows per workgroup: 4 waves x 32
constexpr int kBufferWord3G = 0x00020000;  // raw buffer resource: dword data, bounds-checked
constexpr int kStoreNT = 2;                 // buffer store cache policy: non-temporal

// LDS bytes of one tile (the staged W tile, then one output plane at a time).
template <int K, int N, int NT, int WAVES = 4>
constexpr int gemm_smem_bytes() {
  constexpr int kWBytes = K * (NT * 2 + 16);
  constexpr int kOBytes = WAVES * 32 * (NT * 2 + 16);
  return kWBytes > kOBytes ? kWBytes : kOBytes;
}

// Workgroup -> (head, first row, first column) of its output tile: the tiles
// of head 8 j + x (its column tiles and row blocks) are consecutive
// workgroups on XCD x, so they share the A rows and the weight columns
// through that XCD's L2.
template <int N, int NT, int WAVES>
struct TileCoord {
  int head, r0, n0;
  __device__ __forceinline__ TileCoord(int bid, int R) {
    constexpr int kTilesN = N / NT;
    const int per_head = kTilesN * ((R + WAVES * 32 - 1) / (WAVES * 32));
    const int idx = bid >> 3, inner = idx % per_head;
    head = (idx / per_head) * 8 + (bid & 7);
    n0 = (inner % kTilesN) * NT;
    r0 = (inner / kTilesN) * (WAVES * 32);
  }
};

// The weight tile W[head][0:K][n0:n0+NT] (K rows of NT * 2 bytes): load()
// issues its loads into registers, stage() writes them to LDS (kWPitch bytes
// per k row), where the MFMA loop reads them back transposed as the A operand.
template <int K, int N, int NT, int WAVES>
struct WTile {
  static constexpr int kPitch = NT * 2 + 16;
  static constexpr int kRowChunks = NT / 8;
  static constexpr int kPer = K * kRowChunks / (WAVES * 64);
  static_assert(K * kRowChunks % (WAVES * 64) == 0, "W tile split over the threads");
  u32x4 t[kPer];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ W, int head, int n0) {
    const char* wsrc = reinterpret_cast<const char*>(W + (size_t)head * K * N + n0);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = threadIdx.x + WAVES * 64 * i, k = c / kRowChunks, ch = c % kRowChunks;
      t[i] = *reinterpret_cast<const u32x4*>(wsrc + (size_t)k * N * 2 + ch * 16);
    }
  }
  __device__ __forceinline__ void stage(MLA_LDS char* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = threadIdx.x + WAVES * 64 * i, k = c / kRowChunks, ch = c % kRowChunks;
      *(MLA_LDS u32x4*)(lds + k * kPitch + ch * 16) = t[i];
    }
  }
  // byte offset of this lane's transposed read: k row 16 ks + 8 g + j16/4,
  // column 16*((lane/16)&1) + 4*(j16&3)
  static __device__ __forceinline__ int read_offset(int lane) {
    const int g = lane >> 5, j16 = lane & 15;
    return (8 * g + (j16 >> 2)) * kPitch + (16 * ((lane >> 4) & 1) + 4 * (j16 & 3)) * 2;
  }
  // k-step ks of the transposed product C^T += W^T A^T: `a` holds 8
  // consecutive k (16 ks + 8 g ..) of this lane's row of A
  static __device__ __forceinline__ void kstep(const MLA_LDS char* lds, int w_off, int ks, bf16x8 a,
                                               f32x16 (&c)[NT / 32]) {
    const int o = w_off + 16 * ks * kPitch;
#pragma unroll
    for (int t = 0; t < NT / 32; ++t) {
      const bf16x8 wf = cat4(lds_read_tr4(lds, o + 64 * t), lds_read_tr4(lds, o + 64 * t + 4 * kPitch));
      c[t] = mfma32(wf, a, c[t]);  // C^T tile t: rows = 32 output columns, columns = 32 rows of A
    }
  }
};

// Epilogue of a tile: lane holds C^T[column 32 t + 8 q + 4 g + e][row r32],
// e = 0..3, in c[t][4 q + e]. Each wave stages its own 32 rows in LDS and
// stores them as row segments (only its own LDS rows are read back), first
// the bf16 values, then (with out_lo) in the same rows their rounding
// residues: a wave's LDS operations complete in order, so the residue writes
// follow the reads of the values, and one plane of LDS suffices. The stores
// are non-temporal (cache policy nt): the outputs stream out, and nothing in
// these kernels reads them back. Rows past R are dropped by the buffer bounds.
template <int N, int NT, int WAVES>
__device__ __forceinline__ void store_tile(const f32x16 (&c)[NT / 32], MLA_LDS char* lds,
                                           uint16_t* __restrict__ out, uint16_t* __restrict__ out_lo, int R,
                                           int h, int head, int r0, int n0) {
  constexpr int kOPitch = NT * 2 + 16;  // bytes per staged output row
  constexpr int kNT = NT / 32;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, g = lane >> 5;
  const int orow = wave * 32 + r32;
  constexpr int kLanesPerRow = NT * 2 / 16;
  constexpr int kRowsPerInstr = 64 / kLanesPerRow;
  const int rr = lane / kLanesPerRow, ch = lane % kLanesPerRow;
  const size_t row_stride = (size_t)h * N * 2;  // bytes between consecutive rows of one head
  const int valid = min(WAVES * 32, R - r0);
  const unsigned nbytes = (unsigned)((size_t)(valid - 1) * row_stride + NT * 2);
  // the values go to LDS as they are rounded; their residues wait in
  // registers (32 per lane) until the values have left
  bf16x4 vlo[kNT * 4];
#pragma unroll
  for (int t = 0; t < kNT; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x4 hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = c[t][4 * q + e];
        hi[e] = (__bf16)v;
        vlo[4 * t + q][e] = (__bf16)(v - (float)hi[e]);
      }
      *reinterpret_cast<MLA_LDS bf16x4*>(lds + orow * kOPitch + (32 * t + 8 * q + 4 * g) * 2) = hi;
    }
  auto store_rows = [&](uint16_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(dst + ((size_t)r0 * h + head) * N + n0, 0,
                                                                        nbytes, kBufferWord3G);
#pragma unroll
    for (int k = 0; k < 32; k += kRowsPerInstr) {
      const int lr = wave * 32 + k + rr;
      const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(lds + lr * kOPitch + ch * 16);
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, (unsigned)(lr * row_stride) + ch * 16, 0, kStoreNT);
    }
  };
  store_rows(out);
  if (out_lo != nullptr) {
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<MLA_LDS bf16x4*>(lds + orow * kOPitch + (32 * t + 8 * q + 4 * g) * 2) = vlo[4 * t + q];
    store_rows(out_lo);
  }
}

// One output tile of the per-head GEMM (WAVES x 32 rows), by the workgroup with id `bid`.
template <int K, int N, int NT, int WAVES = 4>
__device__ __forceinline__ void head_gemm_tile(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                               uint16_t* __restrict__ out, uint16_t* __restrict__ out_lo, int R,
                                               int h, int bid, MLA_LDS char* lds) {
  constexpr int kKS = K / 16;  // k-steps
  const TileCoord<N, NT, WAVES> tc(bid, R);
  if (tc.head >= h) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, g = lane >> 5;

  // The W loads go out first and this lane's row of A behind them, so the W
  // tile can be written to LDS (and the first k-steps multiplied) while A
  // still arrives.
  WTile<K, N, NT, WAVES> wt;
  wt.load(W, tc.head, tc.n0);
  // this lane's row of A (padding rows repeat the last row and are never stored)
  const int row = min(tc.r0 + wave * 32 + r32, R - 1);
  const u32x4* arow = reinterpret_cast<const u32x4*>(A + ((size_t)row * h + tc.head) * K) + g;
  bf16x8 af[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) af[ks] = as_bf16x8(arow[2 * ks]);
  wt.stage(lds);
  __syncthreads();

  const int w_off = WTile<K, N, NT, WAVES>::read_offset(lane);
  f32x16 c[NT / 32];
#pragma unroll
  for (int t = 0; t < NT / 32; ++t) c[t] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) WTile<K, N, NT, WAVES>::kstep(lds, w_off, ks, af[ks], c);
  __syncthreads();  // every wave is done reading the W tile
  store_tile<N, NT, WAVES>(c, lds, out, out_lo, R, h, tc.head, tc.r0, tc.n0);
}

template <int K, int N, int NT, int WAVES = 4>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(K == kDNope ? 3 : 1))) void head_gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                        uint16_t* __restrict__ out, uint16_t* __restrict__ out_lo,
                                                        int R, int h) {
  __shared__ __attribute__((aligned(16))) char smem[gemm_smem_bytes<K, N, NT, WAVES>()];
  head_gemm_tile<K, N, NT, WAVES>(A, W, out, out_lo, R, h, blockIdx.x, (MLA_LDS char*)(smem));
}

// The split-KV plan and the query absorption in one launch: the plan reads
// only the cache lengths and the absorption only the queries, so workgroup 0
// plans (mla_plan.h, 256 threads) while the others run the GEMM tiles.
// Workgroups 1..7 have no work; the tiles start at id 8, so that id % 8 is
// still the XCD of a tile. LDS is dynamic: the larger of a tile's and the
// plan's (2 (b + 1) + 5 ints).
constexpr int kPlanWGs = 8;

template <int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void absorb_plan_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ W, uint16_t* __restrict__ out,
                                                          uint16_t* __restrict__ out_lo, int R, int h,
                                                          const int32_t* seqlens, int b, int n_slots, int F,
                                                          int32_t* meta, int32_t* ns_out) {
  extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
  if (blockIdx.x < kPlanWGs) {
    if (blockIdx.x == 0) {
      int* C = reinterpret_cast<int*>(dyn_smem);
      plan_block<256>(seqlens, b, n_slots, F, meta, ns_out, C, C + (b + 1), C + 2 * (b + 1));
    }
    return;
  }
  head_gemm_tile<kDNope, kDLat, NT>(A, W, out, out_lo, R, h, blockIdx.x - kPlanWGs, (MLA_LDS char*)(dyn_smem));
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
  // Narrower column tiles re-read q_nope more often but give more workgroups:
  // that pays with few heads (at h = 32: 7.1 -> 6.2 us), not with 128 heads
  // (14.4 against 16.5 us).
  const int rb = (R + kGemmRows - 1) / kGemmRows;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int hg = (h + 7) / 8 * 8;
  if (h <= 32)
    hipLaunchKernelGGL((head_gemm_kernel<kDNope, kDLat, 64>), dim3(kDLat / 64 * rb * hg), dim3(256), 0, st, q_nope,
                       w_uk, q_lat, q_lat_lo, R, h);
  else
    hipLaunchKernelGGL((head_gemm_kernel<kDNope, kDLat, 128>), dim3(kDLat / 128 * rb * hg), dim3(256), 0, st,
                       q_nope, w_uk, q_lat, q_lat_lo, R, h);
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return clear_error();
}

extern "C" int mla_absorb_q_with_plan(const uint16_t* q_nope, const uint16_t* w_uk, uint16_t* q_lat,
                                      uint16_t* q_lat_lo, int b, int s_q, int h, const int32_t* cache_seqlens,
                                      int num_slots, int split_overhead, int32_t* tile_meta, int32_t* num_splits,
                                      void* stream) {
  const char* fn = "mla_absorb_q_with_plan";
  if (int rc = check_ptr16(fn, q_nope, "q_nope")) return rc;
  if (int rc = check_ptr16(fn, w_uk, "w_uk")) return rc;
  if (int rc = check_ptr16(fn, q_lat, "q_lat")) return rc;
  if (q_lat_lo && reinterpret_cast<uintptr_t>(q_lat_lo) % 16)
    return set_error(MLA_ERR_INVALID_ARG, "%s: q_lat_lo must be 16-byte aligned", fn);
  if (int rc = check_shape(fn, b, s_q, h)) return rc;
  if (int rc = check_plan_args(fn, cache_seqlens, b, num_slots, split_overhead, tile_meta, num_splits)) return rc;
  const int R = b * s_q;
  const int rb = (R + kGemmRows - 1) / kGemmRows;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int hg = (h + 7) / 8 * 8;
  const size_t plan_bytes = sizeof(int) * (2 * ((size_t)b + 1) + 256 / 64 + 1);
  // tile widths as in mla_absorb_q
  const int nt = h <= 32 ? 64 : 128;
  const int tiles = kDLat / nt * rb * hg;
  const size_t smem = std::max(plan_bytes, (size_t)(nt == 64 ? gemm_smem_bytes<kDNope, kDLat, 64>()
                                                             : gemm_smem_bytes<kDNope, kDLat, 128>()));
  // One launch pays only while every workgroup is resident at once: when the
  // tiles already fill the CUs (registers or LDS), the plan's workgroups would
  // push tiles into a second round, so the plan then runs as its own launch
  // ahead of the GEMM (same results).
  int dev = 0, cus = 0, per_cu = 0;
  const void* fused = nt == 64 ? reinterpret_cast<const void*>(absorb_plan_kernel<64>)
                               : reinterpret_cast<const void*>(absorb_plan_kernel<128>);
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0 ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused, 256, smem) != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: cannot query the device", fn);
  if (tiles + kPlanWGs <= (long long)cus * per_cu) {
    if (nt == 64)
      hipLaunchKernelGGL(absorb_plan_kernel<64>, dim3(kPlanWGs + tiles), dim3(256), smem, st, q_nope, w_uk, q_lat,
                         q_lat_lo, R, h, cache_seqlens, b, num_slots, split_overhead, tile_meta, num_splits);
    else
      hipLaunchKernelGGL(absorb_plan_kernel<128>, dim3(kPlanWGs + tiles), dim3(256), smem, st, q_nope, w_uk,
                         q_lat, q_lat_lo, R, h, cache_seqlens, b, num_slots, split_overhead, tile_meta, num_splits);
    if (hipError_t e = hipGetLastError(); e != hipSuccess)
      return set_error(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return clear_error();
  }
  if (int rc = mla_get_metadata(cache_seqlens, b, num_slots, split_overhead, tile_meta, num_splits, stream)) return rc;
  return mla_absorb_q(q_nope, w_uk, q_lat, q_lat_lo, b, s_q, h, stream);
}

extern "C" int mla_up_v(const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o, int b, int s_q, int h,
                        void* stream) {
  const char* fn = "mla_up_v";
  if (int rc = check_ptr16(fn, o_lat, "o_lat")) return rc;
  if (int rc = check_ptr16(fn, w_uv, "w_uv")) return rc;
  if (int rc = check_ptr16(fn, o, "o")) return rc;
  if (int rc = check_shape(fn, b, s_q, h)) return rc;
  const int R = b * s_q;
  // as in mla_absorb_q: narrower tiles with few heads (h = 32: 7.3 -> 6.9 us), not with 128 (11.6 against 16.7 us);
  // with few heads also tiles of 64 rows (two waves), which doubles the workgroups to fill every CU
  // (h = 32, b = 128: 14.1 -> 13.4 us per event-timed call, same outputs)
  const int rb = (R + kGemmRows - 1) / kGemmRows;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int hg = (h + 7) / 8 * 8;
  if (h <= 32) {
    const int rb2 = (R + 63) / 64;
    hipLaunchKernelGGL((head_gemm_kernel<kDLat, kDNope, 32, 2>), dim3(kDNope / 32 * rb2 * hg), dim3(128), 0, st, o_lat,
                       w_uv, o, static_cast<uint16_t*>(nullptr), R, h);
  } else
    hipLaunchKernelGGL((head_gemm_kernel<kDLat, kDNope, 64>), dim3(kDNope / 64 * rb * hg), dim3(256), 0, st, o_lat,
                       w_uv, o, static_cast<uint16_t*>(nullptr), R, h);
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return clear_error();
}
