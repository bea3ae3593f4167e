// Paged MLA decode in the absorbed form (gfx950).
//
// What is computed: for every query row r = (j, i) of sequence b, scores
// s_t = scale * (q_lat[r] . c_t + q_pe[r] . kpe_t) against each visible cached
// token t (the latent c_t and rotated positional key kpe_t share one 576-wide
// row: "DeepSeek-V3 Multi-head Latent Attention (MLA) 深度工程", sections 2.4
// and 3.1), an exact softmax kept in streaming form (the same page's section
// 4.1 recurrence), o_lat[r] = sum_t p_t c_t and lse[r].
//
// How it maps onto MI355X (mla_decode_kernel: one workgroup = NW wavefronts,
// 32 query rows each; with at most 32 rows, mla_decode_tsplit_kernel below
// splits each tile's tokens over four wavefronts instead):
//  * Page loader. A page is 64 rows x 1152 contiguous bytes. It is copied
//    straight from HBM into LDS with 16-byte direct-to-LDS loads
//    (global_load_lds_dwordx4), one wave instruction per 8-row x 128-byte
//    block: 72 instructions per page. Each lane of every instruction reads the
//    same in-block position, so its source address is a per-lane constant
//    plus a per-instruction scalar offset and the loader costs no vector ALU
//    work. Inside a block the 16-byte chunks of row r are XOR-permuted and
//    each 8-row block row is shifted by 32 bytes; with that, the K-fragment
//    reads of QK^T (32 rows x 16 bytes) and the transposed V reads of PV
//    (4 rows x 32 bytes per 16 lanes) both hit 64 distinct banks. Four
//    32-token tile buffers rotate with three tiles in flight, so later tiles
//    stream in while the current one is multiplied; this is the double buffer
//    of the SC11 note's Page Attention figure, done by the CU's own load path
//    instead of separate DMA engines. Rows past the cache length repeat the
//    page's last cached row (finite, and masked to zero weight) and bad page
//    ids read a zero page, so NaN or stale data never reach LDS.
//  * QK^T on the matrix cores, transposed: S^T[token, row] = K Q^T with K
//    (the page rows) as the A operand read from LDS and Q as the B operand
//    held in VGPRs for the whole piece. Each lane then owns 16 scores of ONE
//    query row per 32-token tile, so the row max and row sum are in-lane plus
//    a single exchange between lanes l and l + 32.
//  * The probabilities come out of the score accumulators already in the
//    B-operand layout of the next product, so PV needs no shuffle:
//    O^T[d, row] += V^T P^T, with V^T read from the same LDS page by
//    transposed reads (ds_read_b64_tr_b16). V is columns 0..511 of the row.
//  * Online softmax in base 2 with the scale folded in, against a fixed
//    per-row reference (the row's first tile max) instead of the running
//    max: any reference gives the exact result, fp32 has the range for
//    exp2(x - m_ref) up to 2^64, and the 256 accumulators then never need a
//    rescale (so they stay pinned in AGPRs). A score more than 2^64 above the
//    reference makes the workgroup recompute the piece with a larger one.
//  * Split-KV: the planner hands each workgroup slot a contiguous run of
//    pages (possibly spanning several sequences). A sequence held by one slot
//    is finalised in place; otherwise each piece writes a partial row as fp16
//    divided by its largest magnitude, with that scale and its lse, and
//    mla_combine_kernel merges the pieces by lse rescaling.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "mla_device.h"
#include "mla_host.h"

namespace mla {

__device__ int g_device_error = 0;
__device__ const uint4 g_zero_page[kPage * kRowBytes / 16] = {};  // stands in for a bad page

// LDS page layout (bytes): block (rb, cb) = rows 8rb..8rb+7, chunks 8cb..8cb+7
// sits at rb * kBlkRowStride + cb * 1024; inside it, row r's chunk c is at
// (r % 8) * 128 + ((c % 8) ^ swz(r % 8)) * 16.
constexpr int kBlkBytes = 1024;                              // one wave load instruction
constexpr int kBlkCols = kRowBytes / 128;                    // 9 blocks per 8 rows
constexpr int kBlkRowStride = kBlkCols * kBlkBytes + 32;     // 9248: +32 B rotates banks by 8
constexpr int kTile = 32;                                    // tokens per tile (half a page)
constexpr int kTileStageBytes = (kTile / 8) * kBlkRowStride; // 36992 per tile buffer
constexpr int kStages = 4;                                   // tile buffers in LDS
constexpr int kStageBytes = 2 * kTileStageBytes;             // a whole page (the gather kernel)
constexpr int kRowsBytes8 = 8 * kRowBytes;                   // 9216: 8 cache rows in HBM
constexpr int kQloStride = kDLat * 2 + 16;                   // q_lo rows staged in LDS: 1040 B apart
static_assert(4 * 32 * kQloStride <= kStages * kTileStageBytes, "q_lo staging must fit in the tile buffers");

__device__ __forceinline__ int chunk_swz(int lr) { return ((lr >> 1) & 1) * 4 + (lr >> 2); }
__device__ __forceinline__ int lds_off(int r, int c) {
  return (r >> 3) * kBlkRowStride + (c >> 3) * kBlkBytes + (r & 7) * 128 + (((c & 7) ^ chunk_swz(r & 7)) << 4);
}

constexpr float kLn2 = 0.693147180559945309f;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource: dword data, bounds-checked
constexpr float kRefSlack = 64.0f;  // log2 units a score may exceed the softmax reference


struct DecodeParams {
  const uint16_t* q_lat;
  const uint16_t* q_lat_lo;
  const uint16_t* q_pe;
  const uint16_t* kv;
  const uint8_t* kv8;  // quantised cache (mla_decode_paged_fp8)
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* tile_meta;
  const int32_t* num_splits;
  uint16_t* part_o;   // fp16 bits: partial rows divided by their row scale
  float* part_lse;
  float* part_scale;  // per partial row: largest |value| of the normalised row
  uint16_t* o_lat;
  float* lse;
  long long num_pages;
  int max_blocks, b, s_q, h, log2_h, M, n_rowblocks, num_slots, causal;
  float scale, scale_log2e;
};

__device__ __forceinline__ void flag_error(int bit) { atomicOr(&g_device_error, bit); }

// Read-only plan and table data read at wave-uniform addresses go through the
// scalar cache: nothing in these kernels writes them, so the constant address
// space is valid for the whole launch.
__device__ __forceinline__ int ldc(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Block-table entry of `page` of sequence b (-1 past the table), through the
// scalar cache: consecutive pages of a sequence share a cache line.
__device__ __forceinline__ int fetch_pid(const DecodeParams& P, int b, int page) {
  return page < P.max_blocks ? ldc(P.block_table + (long long)b * P.max_blocks + page) : -1;
}

// Tile loader: one tile (32 tokens, half a page, 4 block rows) of sequence b
// goes to an LDS tile buffer with direct-to-LDS loads; wave w copies block
// rows [w * 4/NW, (w+1) * 4/NW) of it, 9 wave instructions per block row.
// Lane l always fills in-block position l (row l / 8, chunk (l % 8) ^ swz(l / 8)),
// so its HBM address is a uniform page base plus a per-lane 32-bit offset plus
// a uniform block offset. setup() resolves the page; issue(i) sends
// instruction i, so the decode kernel can spread the instructions of a tile
// between its matrix instructions. Rows past the cache length repeat the
// page's last cached row (finite data whose scores the kernel masks, so they
// weigh exactly zero); page ids outside the cache or past the block table
// read a zero page and set the device error word. Every branch is uniform
// (see the note on divergence at the kernel).
template <int NW>
struct TileLoad {
  static constexpr int kRows = 4 / NW;               // block rows per wave
  static constexpr int kInstr = kRows * kBlkCols;    // wave instructions per tile
  const char* base;
  unsigned voff[kRows];
  unsigned dst;  // LDS byte address of the wave's first block row

  __device__ __forceinline__ void setup(const DecodeParams& P, int page, int half, int L, int pid,
                                        MLA_LDS char* stage, int wave, int lane) {
    const bool in_table = page < P.max_blocks;
    const bool ok = in_table && pid >= 0 && pid < P.num_pages;
    if (!ok) flag_error(in_table ? MLA_DEVERR_PAGE_ID : MLA_DEVERR_SEQ_TOO_LONG);
    base = ok ? reinterpret_cast<const char*>(P.kv) + (long long)pid * (kPage * kRowBytes)
              : reinterpret_cast<const char*>(g_zero_page);
    const int last = ok ? min(kPage, L - page * kPage) - 1 : kPage - 1;  // last row to read
    const int lr = lane >> 3, lc = (lane & 7) ^ chunk_swz(lane >> 3);
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int row = half * kTile + (wave * kRows + r) * 8 + lr;  // row within the page
      voff[r] = (unsigned)(min(row, last) * kRowBytes + lc * 16);
    }
    dst = (unsigned)(uintptr_t)(stage + wave * kRows * kBlkRowStride);
  }
  // Not seen by the compiler's wait insertion: callers wait with vmcnt.
  __device__ __forceinline__ void issue(int i) const {
    const int r = i / kBlkCols, cb = i % kBlkCols;
    g2lds16_untracked(base, voff[r] + cb * 128, dst + r * kBlkRowStride + cb * kBlkBytes);
  }
};

// Quantised cache tiles. A page is 64 rows of 640 bytes (512 e4m3 latent
// codes, 64 bf16 key values) and then the 64 fp32 token scales. In LDS a
// 32-token tile keeps the bf16 tile's image layout with 5 blocks of 128 bytes
// per row (the same XOR permutation inside a block, block rows 5152 bytes
// apart), followed by one copy of the page's 64 scales per wave.
constexpr int kRowBytesF = MLA_FP8_ROW_BYTES;               // 640
constexpr int kPageBytesF = MLA_FP8_PAGE_BYTES;             // 41216
constexpr int kScalesOffF = MLA_FP8_SCALES_OFFSET;          // 40960
constexpr int kBlkColsF = kRowBytesF / 128;                 // 5
constexpr int kBlkRowStrideF = kBlkColsF * kBlkBytes + 32;  // 5152
constexpr int kTileDataF = (kTile / 8) * kBlkRowStrideF;    // 20608
constexpr int kTileStageBytesF = kTileDataF + 4 * 256;      // + 4 waves x 64 scales
constexpr int kStagesF = 7;                                 // tile buffers in LDS (6 in flight)
static_assert(kPage * kRowBytes >= kPageBytesF, "the zero page stands in for a quantised page too");

__device__ __forceinline__ int lds_off_f(int r, int c) {
  return (r >> 3) * kBlkRowStrideF + (c >> 3) * kBlkBytes + (r & 7) * 128 + (((c & 7) ^ chunk_swz(r & 7)) << 4);
}

// Loader of one quantised tile for the four waves of mla_decode_tsplit_kernel:
// wave w copies block row w (8 tokens, 5 wave instructions of 1 KB) and the
// page's 64 scales into its own 256-byte copy (one 4-byte load per lane), so
// every wave's own loads cover the scales it reads. Rows past the cache length
// repeat the page's last cached row; page ids outside the cache or past the
// block table read the zero page and set the device error word.
struct TileLoadF {
  static constexpr int kInstr = kBlkColsF + 1;
  const char* base;
  unsigned voff;  // this lane's 16-byte slot in the wave's block row
  unsigned dst;   // LDS byte address of the wave's block row
  unsigned sdst;  // LDS byte address of the wave's scale copy
  unsigned soff;  // this lane's scale

  __device__ __forceinline__ void setup(const DecodeParams& P, int page, int half, int L, int pid,
                                        MLA_LDS char* stage, int wave, int lane) {
    const bool in_table = page < P.max_blocks;
    const bool ok = in_table && pid >= 0 && pid < P.num_pages;
    if (!ok) flag_error(in_table ? MLA_DEVERR_PAGE_ID : MLA_DEVERR_SEQ_TOO_LONG);
    base = ok ? reinterpret_cast<const char*>(P.kv8) + (long long)pid * kPageBytesF
              : reinterpret_cast<const char*>(g_zero_page);
    const int last = ok ? min(kPage, L - page * kPage) - 1 : kPage - 1;
    const int lr = lane >> 3, lc = (lane & 7) ^ chunk_swz(lane >> 3);
    const int row = half * kTile + wave * 8 + lr;
    voff = (unsigned)(min(row, last) * kRowBytesF + lc * 16);
    dst = (unsigned)(uintptr_t)(stage + wave * kBlkRowStrideF);
    sdst = (unsigned)(uintptr_t)(stage + kTileDataF + wave * 256);
    soff = (unsigned)(kScalesOffF + lane * 4);
  }
  __device__ __forceinline__ void issue(int i) const {
    if (i < kBlkColsF) g2lds16_untracked(base, voff + i * 128, dst + i * kBlkBytes);
    else g2lds4_untracked(base, soff, sdst);
  }
};

// Workgroup barrier of the tile pipeline. The wave's LDS operations finish
// first; its direct-to-LDS loads of later tiles stay in flight (each wave has
// already waited for its share of the tile the barrier publishes). A fenced
// __syncthreads would wait for those loads too.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt for vector memory only (expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Divergence note: the kernel keeps every branch wave-uniform. Register
// pressure makes the compiler park live values (row index, pointers) in spare
// registers around the epilogue, and a reload placed inside a lane-masked
// region restores only the active lanes; with no lane-masked regions every
// reload covers the whole wave. Padding rows are handled by bounds-checked
// buffer stores and source selects instead of branches.
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_kernel(DecodeParams P) {
  __shared__ __attribute__((aligned(16))) char smem[kStages * kTileStageBytes];
  // restart request of the current pass: cleared when a pass starts, set by
  // any wave whose scores outgrow the reference, read by all after the pass
  __shared__ int restart_flag;
  MLA_LDS char* lds = (MLA_LDS char*)(smem);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int r32 = lane & 31;
  const int g = lane >> 5;

  // workgroup -> (slot, row block); the row blocks of one slot share an XCD
  int slot, rb;
  {
    const int R = P.n_rowblocks;
    const int bid = blockIdx.x;
    if (R == 1) {
      slot = bid;
      rb = 0;
    } else {
      const int xcd = bid & 7, idx = bid >> 3;
      slot = (idx / R) * 8 + xcd;
      rb = idx % R;
    }
  }
  if (slot >= P.num_slots) return;
  const int* meta = P.tile_meta + slot * MLA_META_WORDS;
  const int b_begin = ldc(meta + 0), page_begin = ldc(meta + 1), b_end = ldc(meta + 2), page_end = ldc(meta + 3);
  const int split_begin = ldc(meta + 4);
  if (b_end < b_begin) return;

  const int M = P.M;
  const int row = rb * (NW * 32) + wave * 32 + r32;  // query row within the sequence
  // padding rows alias the last row: they repeat its work (so they raise no
  // restart of their own) and are never stored
  const int row_c = min(row, M - 1);
  const int qj = row_c >> P.log2_h;                  // query token index of this row (h is a power of 2)
  const bf16x8 zero8 = bf16x8{};
  // Tiles in flight: while tile j is multiplied, the loads of tile j + kAhead
  // go out between its matrix instructions (kAhead + 1 <= kStages buffers).
  constexpr int kNLd = TileLoad<NW>::kInstr;
  constexpr int kAhead = NW == 1 ? 2 : 3;  // keeps the outstanding count within vmcnt's 63
  static_assert((kAhead - 1) * kNLd < 64 && kAhead < kStages, "load pipeline depth");

  // LDS-relative constants of this lane (see the layout at kBlkRowStride).
  // K fragment for k-step ks of a 32-token tile: token r32, chunk 2 ks + g
  //   -> a_base[ks % 4] + (ks / 4) * 1024.
  int a_base[4];
  {
    const int lr = r32 & 7;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
      a_base[k4] = (r32 >> 3) * kBlkRowStride + lr * 128 + (((2 * k4 + g) ^ chunk_swz(lr)) << 4);
  }
  // V^T fragment (transposed read) for d-tile dt and k-step kk of a tile:
  //   rows 16 kk + 4 g + j/4 (+8 for the second read), byte column
  //   64 dt + 32 ((lane/16) & 1) + 8 (j & 3)
  //   -> v_base[dt % 2] + (dt / 2) * 1024 + 2 kk * kBlkRowStride (+ kBlkRowStride).
  int v_base[2];
  {
    const int j16 = lane & 15;
    const int lr = 4 * g + (j16 >> 2);
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2)
      v_base[p2] = lr * 128 + (((4 * p2 + 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1)) ^ chunk_swz(lr)) << 4) +
                   8 * (j16 & 1);
  }

  for (int b = b_begin; b <= b_end; ++b) {
    // Per-lane values used by a piece are rebuilt from the lane id here (the
    // empty asm hides that it is loop invariant): kept across pieces they
    // were spilled, and a reload waits for every outstanding load.
    int pl = lane;
    asm volatile("" : "+v"(pl));
    const int pr32 = pl & 31, pg = pl >> 5;
    const int prow_c = min(rb * (NW * 32) + wave * 32 + pr32, M - 1);
    const int pqj = prow_c >> P.log2_h;
    const int L = ldc(P.seqlens + b);
    const int npages = L > 0 ? (L + kPage - 1) / kPage : 0;
    const int p_lo = (b == b_begin) ? page_begin : 0;
    const int p_hi = (b == b_end) ? page_end : npages;
    if (p_hi <= p_lo) continue;
    const int ns0 = ldc(P.num_splits + b), ns1 = ldc(P.num_splits + b + 1);
    const int split = (b == b_begin) ? split_begin : ns0;
    const bool single = (ns1 - ns0) == 1;
    const int n_row = P.causal ? L - P.s_q + 1 + pqj : L;  // keys this row sees
    const int n_min = P.causal ? L - P.s_q + 1 : L;       // fewest keys of any row

    const int tok0 = p_lo * kPage;
    const int n_tiles = (min(p_hi * kPage, L) - tok0 + kTile - 1) / kTile;  // tiles holding cached tokens
    bf16x8 qf[36];
    {
      // Buffer loads: a uniform base per sequence plus a 32-bit lane offset
      // that is rebuilt here (the empty asm hides that it is loop invariant).
      // A hoisted 64-bit per-lane pointer would be spilled, and reloading it
      // between the loads made the wave wait for all of them first.
      const int qr = prow_c;
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(P.q_lat + (long long)b * M * kDLat), 0, M * kDLat * 2, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(P.q_pe + (long long)b * M * kDRope), 0, M * kDRope * 2, kBufferWord3);
      const int oq = qr * (kDLat * 2) + 16 * pg, op = qr * (kDRope * 2) + 16 * pg;
#pragma unroll
      for (int ks = 0; ks < 32; ++ks)
        qf[ks] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rq, oq + 32 * ks, 0, 0));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[32 + ks] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rp, op + 32 * ks, 0, 0));
    }

    // Softmax reference. Probabilities are exp2(x - m_ref) with m_ref fixed
    // for the whole piece, so the accumulators never need rescaling; m_ref is
    // the row's first finite tile max. If a later score exceeds it by more
    // than kRefSlack (where fp32 sums could start to overflow), the whole
    // workgroup runs the piece again with the row max of the first pass.
    float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
    f32x16 acc[16];
    TileLoad<NW> ld;
    int pid = -1;  // page id of the last tile set up
    // The first tiles go out right behind the query loads, so both arrive
    // in one memory round trip.
    auto issue_first_tiles = [&]() {
#pragma unroll 1
      for (int t = 0; t < min(kAhead, n_tiles); ++t) {
        if ((t & 1) == 0) pid = fetch_pid(P, b, p_lo + (t >> 1));
        ld.setup(P, p_lo + (t >> 1), t & 1, L, pid, lds + (t % kStages) * kTileStageBytes, wave, pl);
#pragma unroll
        for (int i = 0; i < kNLd; ++i) ld.issue(i);
      }
    };
    __syncthreads();   // every wave is done with the LDS use of the previous piece
    restart_flag = 0;  // every lane writes 0
    issue_first_tiles();
    for (;;) {  // restart loop: runs once unless a score outgrows m_ref
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) mfma32_agpr_zero(acc[dt], zero8);
      m_ref = m_seen;
      l_run = 0.f;
      for (int j = 0; j < n_tiles; ++j) {
        // this wave's loads of tile j are done once at most the later tiles'
        // remain; the barrier then covers every wave's share
        const int later = min(kAhead - 1, n_tiles - 1 - j);
        if (later >= 2) wait_vmcnt<kAhead >= 3 ? 2 * kNLd : 0>();
        else if (later == 1) wait_vmcnt<kNLd>();
        else wait_vmcnt<0>();
        barrier_keep_loads();
        const bool more = j + kAhead < n_tiles;
        if (more) {  // tile j + kAhead reuses the buffer of tile j - 1
          const int t = j + kAhead;
          ld.setup(P, p_lo + (t >> 1), t & 1, L, pid, lds + (t % kStages) * kTileStageBytes, wave, pl);
        }
        __builtin_amdgcn_sched_barrier(0);
        MLA_LDS char* tile = lds + (j % kStages) * kTileStageBytes;
        // load instruction slots: the 68 matrix instructions of a tile carry
        // the kNLd loads of tile j + kAhead, evenly spaced
#define MLA_LOAD_SLOT(m)                                                          \
  if ((((m) + 1) * kNLd) / 68 != ((m) * kNLd) / 68 && more) ld.issue(((m) * kNLd) / 68);

        // ---- S^T = K Q^T (576 deep), fragments read four k-steps ahead ----
        // the sched barriers keep the scheduler from hoisting every fragment
        // read (they would not fit in VGPRs)
        f32x16 sc = f32x16{};
        {
          bf16x8 kr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) kr[i] = lds_read16(tile, a_base[i]);
#pragma unroll
          for (int ks = 0; ks < 36; ++ks) {
            sc = mfma32(kr[ks & 3], qf[ks], sc);
            if (ks + 4 < 36) kr[ks & 3] = lds_read16(tile, a_base[(ks + 4) & 3] + ((ks + 4) >> 2) * kBlkBytes);
            MLA_LOAD_SLOT(ks)
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        // ---- softmax numerators, base 2 ----
        // sc element v is token tok0 + 32 j + 8 (v / 4) + 4 g + v % 4
        const int t0 = tok0 + j * kTile + 4 * pg;
        if (tok0 + j * kTile + kTile > n_min) {  // some token of this tile is masked for some row
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (t0 + 8 * (v >> 2) + (v & 3) >= n_row) sc[v] = -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * P.scale_log2e;  // scale > 0 commutes with max
        m_seen = fmaxf(m_seen, mx);
        if (m_ref == -INFINITY) m_ref = mx;  // nothing accumulated yet for this row
        if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRefSlack) != 0ull) restart_flag = 1;
        const float msub = m_ref == -INFINITY ? 0.f : m_ref;
        float psum = 0.f;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          sc[v] = fast_exp2(sc[v] * P.scale_log2e - msub);
          psum += sc[v];
        }
        const bf16x8 pb0 = pack8(sc[0], sc[1], sc[2], sc[3], sc[4], sc[5], sc[6], sc[7]);
        bf16x8 pb1;

        // ---- O^T += V^T P^T over this tile's 32 tokens, fragments four steps ahead ----
        // k-step major (it = kk * 16 + dt): the first 16 matrix instructions
        // need only the first 8 probabilities, and the other 8 are computed
        // between them
        {
          bf16x4 vr[4][2];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int o = v_base[i & 1] + (i >> 1) * kBlkBytes;
            vr[i][0] = lds_read_tr4(tile, o);
            vr[i][1] = lds_read_tr4(tile, o + kBlkRowStride);
          }
#pragma unroll
          for (int it = 0; it < 32; ++it) {
            const int dt = it & 15, kk = it >> 4;
            if (it == 16) pb1 = pack8(sc[8], sc[9], sc[10], sc[11], sc[12], sc[13], sc[14], sc[15]);
            mfma32_agpr(acc[dt], cat4(vr[it & 3][0], vr[it & 3][1]), kk ? pb1 : pb0);
            if (it < 8) {
              sc[8 + it] = fast_exp2(sc[8 + it] * P.scale_log2e - msub);
              psum += sc[8 + it];
            }
            if (it + 4 < 32) {
              const int n = it + 4, ndt = n & 15, nkk = n >> 4;
              const int o = v_base[ndt & 1] + (ndt >> 1) * kBlkBytes + 2 * nkk * kBlkRowStride;
              vr[it & 3][0] = lds_read_tr4(tile, o);
              vr[it & 3][1] = lds_read_tr4(tile, o + kBlkRowStride);
            }
            MLA_LOAD_SLOT(36 + it)
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        l_run += psum;
#undef MLA_LOAD_SLOT
        // page id of the tile the next iteration sets up, fetched here so
        // that its latency passes under the barrier
        {
          const int tn = j + 1 + kAhead;
          if (tn < n_tiles && (tn & 1) == 0) pid = fetch_pid(P, b, p_lo + (tn >> 1));
        }
      }
      wait_vmem_all();
      __syncthreads();
      if (restart_flag == 0) break;
      // a score outgrew the reference: the pass ran to its end (its sums may
      // have overflowed) and m_seen is now the row's true max, so the next
      // pass cannot restart again
      __syncthreads();  // every wave has read the flag
      restart_flag = 0;
      issue_first_tiles();
    }
    mfma_drain();

    // ---- finalise this piece ----
    // Stores go through buffer resources sized to the valid rows of this row
    // block: lanes of padding rows get offsets past the end and the hardware
    // drops their writes, so no lane is masked off by a branch.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float lse_v = l_tot > 0.f ? (m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
    const int row0 = rb * (NW * 32);                  // first row of this row block
    if (single && P.q_lat_lo != nullptr) {
      // The scores used q_lat rounded to bf16; the residue q_lo = q_lat - bf16(q_lat)
      // shifts score t by scale * (q_lo . c_t). lse is smooth in the scores with
      // d lse / d s_t = p_t, so to first order lse moves by
      // scale * sum_t p_t (q_lo . c_t) = scale * (q_lo . o_lat): one 512-long dot
      // per row instead of a second pass over every token. The dropped second
      // order term is at most half the square of the largest shift (~1e-5).
      // Split pieces leave this to mla_combine, which applies it to the merged row.
      // The wave's 32 q_lo rows go to LDS (both page buffers are idle after the
      // piece's last barrier), kQloStride apart so the 8-byte reads spread over
      // the banks; each lane then reads the values that match its accumulators.
      MLA_LDS char* qs = lds + wave * (32 * kQloStride);
      const char* src = reinterpret_cast<const char*>(P.q_lat_lo) + pl * 16;
#pragma unroll 4
      for (int i = 0; i < 32; ++i) {
        const long long r = (long long)b * M + min(row0 + wave * 32 + i, M - 1);
        g2lds16(src + r * (kDLat * 2), qs + i * kQloStride);
      }
      wait_vmem_all();
      const MLA_LDS char* qrow_l = qs + pr32 * kQloStride + 8 * pg;
      float dot = 0.f;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const bf16x4 q4 = *reinterpret_cast<const MLA_LDS bf16x4*>(qrow_l + 64 * dt + 16 * vq);  // d = 32 dt + 8 vq + 4 g
#pragma unroll
          for (int e = 0; e < 4; ++e) dot += acc[dt][4 * vq + e] * (float)q4[e];
        }
      dot += __shfl_xor(dot, 32);
      if (l_tot > 0.f) lse_v += P.scale * dot * inv_l;
    }
    const int nrows = min(NW * 32, M - row0);         // valid rows in it
    const int lrow = wave * 32 + pr32;                // this lane's row within the block
    // Rows leave through LDS: each lane holds 4-value pieces of one row, so
    // direct stores would write 32 rows x 32 bytes per instruction. The wave
    // puts its 32 rows into its own LDS rows (kQloStride apart, so the
    // writes of 16 rows hit distinct banks), then every store instruction
    // writes one whole contiguous row piece of 1 KB. Only this wave touches
    // its LDS rows and one wave's LDS operations complete in order, so no
    // barrier is needed; the tile buffers are idle after the piece's last
    // barrier. Buffer resources sized to the valid rows drop the writes of
    // padding rows.
    MLA_LDS char* tw = lds + wave * (32 * kQloStride);
    const int wr = pr32 * kQloStride;  // this lane's row in the wave's LDS rows
    if (single) {
      const long long rbase = (long long)b * M + row0;
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          P.o_lat + rbase * kDLat, 0, nrows * kDLat * 2, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(P.lse + rbase, 0, nrows * 4,
                                                                          kBufferWord3);
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {  // d = 32 dt + 8 vq + 4 g + e
          bf16x4 w;
          w[0] = (__bf16)(acc[dt][4 * vq + 0] * inv_l);
          w[1] = (__bf16)(acc[dt][4 * vq + 1] * inv_l);
          w[2] = (__bf16)(acc[dt][4 * vq + 2] * inv_l);
          w[3] = (__bf16)(acc[dt][4 * vq + 3] * inv_l);
          *reinterpret_cast<MLA_LDS bf16x4*>(tw + wr + (dt * 32 + 8 * vq + 4 * pg) * 2) = w;
        }
#pragma unroll 8
      for (int k = 0; k < 32; ++k) {  // row wave * 32 + k: 64 lanes x 16 bytes
        const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(tw + k * kQloStride + pl * 16);
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, (wave * 32 + k) * (kDLat * 2) + pl * 16, 0, 0);
      }
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse_v), rl, lrow * 4, 0, 0);
    } else {
      // Split pieces publish fp16 rows scaled by their largest magnitude
      // (values in [-1, 1], 11 significant bits: half the bytes of fp32 for
      // the same merged result within rounding) plus the scale and lse.
      const long long pbase = (long long)split * M + row0;
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          P.part_o + pbase * kDLat, 0, nrows * kDLat * 2, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(P.part_lse + pbase, 0, nrows * 4,
                                                                          kBufferWord3);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(P.part_scale + pbase, 0, nrows * 4,
                                                                          kBufferWord3);
      float amax = 0.f;  // row max of |O| (the lane pair l, l + 32 holds one row)
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(acc[dt][v]));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const float mul = amax > 0.f ? 1.f / amax : 0.f;
      const float row_scale = amax * inv_l;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {  // d = 32 dt + 8 vq + 4 g + e
          _Float16 w0 = (_Float16)(acc[dt][4 * vq + 0] * mul), w1 = (_Float16)(acc[dt][4 * vq + 1] * mul);
          _Float16 w2 = (_Float16)(acc[dt][4 * vq + 2] * mul), w3 = (_Float16)(acc[dt][4 * vq + 3] * mul);
          u32x2 w;
          w[0] = (unsigned)__builtin_bit_cast(unsigned short, w0) | ((unsigned)__builtin_bit_cast(unsigned short, w1) << 16);
          w[1] = (unsigned)__builtin_bit_cast(unsigned short, w2) | ((unsigned)__builtin_bit_cast(unsigned short, w3) << 16);
          *reinterpret_cast<MLA_LDS u32x2*>(tw + wr + (dt * 32 + 8 * vq + 4 * pg) * 2) = w;
        }
#pragma unroll 8
      for (int k = 0; k < 32; ++k) {  // row wave * 32 + k: 64 lanes x 16 bytes
        const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(tw + k * kQloStride + pl * 16);
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, (wave * 32 + k) * (kDLat * 2) + pl * 16, 0, 0);
      }
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, row_scale), rs, lrow * 4, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse_v), rl, lrow * 4, 0, 0);
    }
  }
}

// Token-split decode for one block of at most 32 query rows (M <= 32: one
// tensor-parallel share of the heads, or few heads). One row block gives one
// wave nothing to share a tile with, so here the four waves of the workgroup
// split every 32-token tile instead: wave (th, rh) = (wave % 2, wave / 2)
// scores tokens 16 th .. 16 th + 15 of the tile against rows 16 rh .. 16 rh + 15
// (16x16x32 MFMAs, K from the same LDS tile image, Q in registers), writes its
// probabilities to a small LDS buffer, and after a barrier every wave
// accumulates its own 128 columns of o_lat for all 32 rows from the whole
// tile (O^T = V^T P^T as in mla_decode_kernel). The loader, the tile
// pipeline, the fixed softmax reference with restart and the epilogue
// formats are those of mla_decode_kernel; the reference of a row is shared by
// the two waves that score it (exchanged once per piece through LDS).
// With kFp8 the cache is the quantised page format: tiles are half as large
// (seven buffers, six tiles in flight), the K and V fragments of the latent
// part are e4m3 codes widened to bf16 in registers (exactly), each token's
// scale multiplies its latent dot product before the positional part is added,
// and the probabilities that weight its latent row carry the scale too. With
// power-of-two scales this is, rounding step for rounding step, the bf16
// kernel on the dequantised cache.
template <bool kFp8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_tsplit_kernel(DecodeParams P) {
  constexpr int kStg = kFp8 ? kStagesF : kStages;
  constexpr int kStgBytes = kFp8 ? kTileStageBytesF : kTileStageBytes;
  __shared__ __attribute__((aligned(16))) char smem[kStg * kStgBytes];
  __shared__ __attribute__((aligned(16))) char pbuf[2 * 32 * 32];  // P^T: [k-step][row][16 tokens] bf16 (permuted)
  __shared__ float xmax[4][16];  // per-wave row maxima (reference and restart exchanges)
  __shared__ float xl[4][16];    // per-wave row sums
  __shared__ float xm[2][16];    // the reference of each row
  __shared__ float xred[4][32];  // per-wave partial row dots / maxima in the epilogue
  __shared__ int restart_flag;
  MLA_LDS char* lds = (MLA_LDS char*)(smem);
  MLA_LDS char* pb = (MLA_LDS char*)(pbuf);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int th = wave & 1, rh = wave >> 1;
  const int slot = blockIdx.x;
  if (slot >= P.num_slots) return;
  const int* meta = P.tile_meta + slot * MLA_META_WORDS;
  const int b_begin = ldc(meta + 0), page_begin = ldc(meta + 1), b_end = ldc(meta + 2), page_end = ldc(meta + 3);
  const int split_begin = ldc(meta + 4);
  if (b_end < b_begin) return;
  const int M = P.M;
  using Loader = std::conditional_t<kFp8, TileLoadF, TileLoad<4>>;
  constexpr int kNLd = Loader::kInstr;       // loads per wave per tile: 9 (bf16) or 6 (quantised)
  constexpr int kAhead = kFp8 ? 6 : 3;       // tiles in flight
  static_assert((kAhead - 1) * kNLd < 64 && kAhead < kStg, "load pipeline depth");
  constexpr int kSlots = 18 + 8;             // matrix instructions per tile and wave

  // K fragment (A operand) of k-step ks: token 16 th + l % 16 of the tile,
  // 16-byte chunk 4 ks + l / 16 -> ka[ks % 2] + (ks / 2) * 1024.
  int ka[2];
  {
    const int r = 16 * th + (lane & 15), lr = r & 7;
#pragma unroll
    for (int p = 0; p < 2; ++p)
      ka[p] = (r >> 3) * kBlkRowStride + lr * 128 + (((4 * p + (lane >> 4)) ^ chunk_swz(lr)) << 4);
  }
  // Quantised tiles: the latent fragment of k-step ks (< 16) is 8 codes of
  // token 16 th + l % 16 at row byte 32 ks + 8 (l / 16): 16-byte chunk
  // 2 ks + l / 32, half (l / 16) % 2 -> kl[ks % 4] + (ks / 4) * 1024. The
  // positional fragments (k-steps 16, 17) are bf16 in the row's fifth block.
  int kl[4], kp[2];
  if constexpr (kFp8) {
    const int r = 16 * th + (lane & 15), lr = r & 7, lg = lane >> 4;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      kl[q] = (r >> 3) * kBlkRowStrideF + lr * 128 + (((2 * q + (lg >> 1)) ^ chunk_swz(lr)) << 4) + 8 * (lg & 1);
#pragma unroll
    for (int p = 0; p < 2; ++p)
      kp[p] = (r >> 3) * kBlkRowStrideF + 4 * kBlkBytes + lr * 128 + (((4 * p + lg) ^ chunk_swz(lr)) << 4);
  }
  // V^T fragment of this wave's d-tile dt (global d-tile 4 wave + dt) and k-step kk:
  //   v_base[dt % 2] + (2 wave + dt / 2) * 1024 + 2 kk * kBlkRowStride (+ kBlkRowStride)
  int v_base[2];
  {
    const int j16 = lane & 15, g = lane >> 5;
    const int lr = 4 * g + (j16 >> 2);
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2)
      v_base[p2] = lr * 128 + (((4 * p2 + 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1)) ^ chunk_swz(lr)) << 4) +
                   8 * (j16 & 1) + wave * 2048;
  }
  // Quantised tiles: V^T fragment of d-tile dt (d = 128 wave + 32 dt + l % 32)
  // and k-step kk by one 8-bit transposed read. Its 8 tokens must be those of
  // the bf16 fragment, in the same order (the k order P^T is stored in): lane
  // group g = l / 32 holds tokens 16 kk + 4 g + {0, 1, 2, 3, 8, 9, 10, 11}. The
  // k-th byte a lane receives comes from the row that lanes 2 k and 2 k + 1 of
  // its 16-lane block B address, so lane j of block B addresses token
  // 16 kk + 4 (B / 2) + (j / 2) % 4 + 8 (j / 8) at row byte
  // 128 wave + 32 dt + 16 (B % 2) + 8 (j % 2)  ->  vf[dt] + 2 kk * kBlkRowStrideF
  int vf[4];
  if constexpr (kFp8) {
    const int B = lane >> 4, j = lane & 15;
    const int lr = 4 * (B >> 1) + ((j >> 1) & 3);  // token within its 8-token block row
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      vf[dt] = (j >> 3) * kBlkRowStrideF + wave * kBlkBytes + lr * 128 +
               (((2 * dt + (B & 1)) ^ chunk_swz(lr)) << 4) + 8 * (j & 1);
  }

  for (int b = b_begin; b <= b_end; ++b) {
    const int L = ldc(P.seqlens + b);
    const int npages = L > 0 ? (L + kPage - 1) / kPage : 0;
    const int p_lo = (b == b_begin) ? page_begin : 0;
    const int p_hi = (b == b_end) ? page_end : npages;
    if (p_hi <= p_lo) continue;
    const int ns0 = ldc(P.num_splits + b), ns1 = ldc(P.num_splits + b + 1);
    const int split = (b == b_begin) ? split_begin : ns0;
    const bool single = (ns1 - ns0) == 1;
    // this lane's query row in the score product (padding rows alias row M - 1)
    const int qrow = min(16 * rh + (lane & 15), M - 1);
    const int n_row = P.causal ? L - P.s_q + 1 + (qrow >> P.log2_h) : L;  // keys this row sees
    const int n_min = P.causal ? L - P.s_q + 1 : L;                      // fewest keys of any row
    const int tok0 = p_lo * kPage;
    const int n_tiles = (min(p_hi * kPage, L) - tok0 + kTile - 1) / kTile;

    bf16x8 qf[18];  // B operand: row qrow, dims 32 ks + 8 (l / 16) .. + 7
    {
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(P.q_lat + (long long)b * M * kDLat), 0, M * kDLat * 2, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(P.q_pe + (long long)b * M * kDRope), 0, M * kDRope * 2, kBufferWord3);
      const int oq = qrow * (kDLat * 2) + 16 * (lane >> 4), op = qrow * (kDRope * 2) + 16 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        qf[ks] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rq, oq + 64 * ks, 0, 0));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        qf[16 + ks] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rp, op + 64 * ks, 0, 0));
    }

    float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
    f32x16 acc[4];
    Loader ld;
    int pid = -1;
    auto issue_first_tiles = [&]() {
#pragma unroll 1
      for (int t = 0; t < min(kAhead, n_tiles); ++t) {
        if ((t & 1) == 0) pid = fetch_pid(P, b, p_lo + (t >> 1));
        ld.setup(P, p_lo + (t >> 1), t & 1, L, pid, lds + (t % kStg) * kStgBytes, wave, lane);
#pragma unroll
        for (int i = 0; i < kNLd; ++i) ld.issue(i);
      }
    };
    __syncthreads();  // every wave is done with the LDS use of the previous piece
    restart_flag = 0;
    issue_first_tiles();
    for (int pass = 0;; ++pass) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
      m_ref = m_seen;
      l_run = 0.f;
      for (int j = 0; j < n_tiles; ++j) {
        const int later = min(kAhead - 1, n_tiles - 1 - j);  // this wave's later tiles still loading
        switch (later) {  // uniform
          case 5: wait_vmcnt<(kAhead > 5 ? 5 * kNLd : 0)>(); break;
          case 4: wait_vmcnt<(kAhead > 4 ? 4 * kNLd : 0)>(); break;
          case 3: wait_vmcnt<(kAhead > 3 ? 3 * kNLd : 0)>(); break;
          case 2: wait_vmcnt<2 * kNLd>(); break;
          case 1: wait_vmcnt<kNLd>(); break;
          default: wait_vmcnt<0>(); break;
        }
        barrier_keep_loads();
        const bool more = j + kAhead < n_tiles;
        if (more) {
          const int t = j + kAhead;
          if ((t & 1) == 0) pid = fetch_pid(P, b, p_lo + (t >> 1));
          ld.setup(P, p_lo + (t >> 1), t & 1, L, pid, lds + (t % kStg) * kStgBytes, wave, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        MLA_LDS char* tile = lds + (j % kStg) * kStgBytes;
#define MLA_TS_LOAD_SLOT(m) \
  if ((((m) + 1) * kNLd) / kSlots != ((m) * kNLd) / kSlots && more) ld.issue(((m) * kNLd) / kSlots);

        // ---- S^T = K Q^T for 16 tokens x 16 rows, 576 deep ----
        f32x4 sc = f32x4{};
        f32x4 tsc;  // quantised tiles: the scales of this lane's 4 tokens
        if constexpr (kFp8) {
          // codes read four k-steps ahead, widened one k-step ahead (under the
          // running matrix instruction)
          u32x2 kr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) kr[i] = lds_read8(tile, kl[i]);
          bf16x8 kb = fp8x8_to_bf16(kr[0]);
#pragma unroll
          for (int ks = 0; ks < 16; ++ks) {
            const bf16x8 cur = kb;
            sc = mfma16(cur, qf[ks], sc);
            if (ks + 1 < 16) kb = fp8x8_to_bf16(kr[(ks + 1) & 3]);
            if (ks + 4 < 16) kr[ks & 3] = lds_read8(tile, kl[(ks + 4) & 3] + ((ks + 4) >> 2) * kBlkBytes);
            MLA_TS_LOAD_SLOT(ks)
            __builtin_amdgcn_sched_barrier(0);
          }
          // the latent dot products carry each token's scale; then the positional part
          tsc = *reinterpret_cast<const MLA_LDS f32x4*>(tile + kTileDataF + wave * 256 +
                                                        ((j & 1) * kTile + 16 * th + 4 * (lane >> 4)) * 4);
          const bf16x8 r0 = lds_read16(tile, kp[0]), r1 = lds_read16(tile, kp[1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[i] *= tsc[i];
          sc = mfma16(r0, qf[16], sc);
          MLA_TS_LOAD_SLOT(16)
          __builtin_amdgcn_sched_barrier(0);
          sc = mfma16(r1, qf[17], sc);
          MLA_TS_LOAD_SLOT(17)
          __builtin_amdgcn_sched_barrier(0);
        } else {
          bf16x8 kr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) kr[i] = lds_read16(tile, ka[i & 1] + (i >> 1) * kBlkBytes);
#pragma unroll
          for (int ks = 0; ks < 18; ++ks) {
            sc = mfma16(kr[ks & 3], qf[ks], sc);
            if (ks + 4 < 18) kr[ks & 3] = lds_read16(tile, ka[(ks + 4) & 1] + ((ks + 4) >> 1) * kBlkBytes);
            MLA_TS_LOAD_SLOT(ks)
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        // ---- softmax numerators, base 2; sc[i] is token 16 th + 4 (l / 16) + i ----
        const int t0 = tok0 + j * kTile + 16 * th + 4 * (lane >> 4);
        if (tok0 + j * kTile + kTile > n_min) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + i >= n_row) sc[i] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * P.scale_log2e;  // this wave's 16 tokens of the row
        m_seen = fmaxf(m_seen, mx);
        if (pass == 0 && j == 0) {
          // the reference is the row's max over the whole first tile: both
          // halves of the tile take it from each other
          xmax[wave][lane & 15] = mx;
          barrier_keep_loads();
          m_ref = fmaxf(mx, xmax[wave ^ 1][lane & 15]);
        }
        if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRefSlack) != 0ull) restart_flag = 1;
        const float msub = m_ref == -INFINITY ? 0.f : m_ref;
        bf16x4 pw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(sc[i] * P.scale_log2e - msub);
          l_run += p;
          // quantised tiles: the weight of the token's latent row carries its
          // scale (a masked token weighs 0 whatever its scale slot holds)
          if constexpr (kFp8) pw[i] = (__bf16)(p > 0.f ? p * tsc[i] : 0.f);
          else pw[i] = (__bf16)p;
        }
        // P^T of k-step th, row 16 rh + l % 16, stored in the k order of the
        // V^T fragments (lane group g of a fragment holds tokens 4 g .. 4 g + 3
        // and 8 + 4 g .. 8 + 4 g + 3): token t sits at byte
        // 16 ((t / 4) % 2) + 8 (t / 8) + 2 (t % 4) of the row's 32 bytes
        *reinterpret_cast<MLA_LDS bf16x4*>(pb + th * 1024 + (16 * rh + (lane & 15)) * 32 +
                                           ((lane >> 4) & 1) * 16 + (lane >> 5) * 8) = pw;
        barrier_keep_loads();

        // ---- O^T += V^T P^T: this wave's 128 columns, all 32 rows, 32 tokens ----
        if constexpr (kFp8) {
          bf16x8 pf[2];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) pf[kk] = lds_read16(pb, kk * 1024 + (lane & 31) * 32 + (lane >> 5) * 16);
          u32x2 vq[8];
#pragma unroll
          for (int it = 0; it < 8; ++it) vq[it] = lds_read_tr8(tile, vf[it >> 1] + 2 * (it & 1) * kBlkRowStrideF);
          bf16x8 vb = fp8x8_to_bf16(vq[0]);
#pragma unroll
          for (int it = 0; it < 8; ++it) {  // it = dt * 2 + kk; widened one step ahead
            const int dt = it >> 1, kk = it & 1;
            const bf16x8 cur = vb;
            acc[dt] = mfma32(cur, pf[kk], acc[dt]);
            if (it + 1 < 8) vb = fp8x8_to_bf16(vq[it + 1]);
            MLA_TS_LOAD_SLOT(18 + it)
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          bf16x8 pf[2];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) pf[kk] = lds_read16(pb, kk * 1024 + (lane & 31) * 32 + (lane >> 5) * 16);
          bf16x4 vr[8][2];
#pragma unroll
          for (int it = 0; it < 8; ++it) {  // it = dt * 2 + kk
            const int dt = it >> 1, kk = it & 1;
            const int o = v_base[dt & 1] + (dt >> 1) * kBlkBytes + 2 * kk * kBlkRowStride;
            vr[it][0] = lds_read_tr4(tile, o);
            vr[it][1] = lds_read_tr4(tile, o + kBlkRowStride);
          }
#pragma unroll
          for (int it = 0; it < 8; ++it) {
            const int dt = it >> 1, kk = it & 1;
            acc[dt] = mfma32(cat4(vr[it][0], vr[it][1]), pf[kk], acc[dt]);
            MLA_TS_LOAD_SLOT(18 + it)
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#undef MLA_TS_LOAD_SLOT
      }
      wait_vmem_all();
      __syncthreads();
      if (restart_flag == 0) break;
      // a score outgrew the reference: rerun with the row's true max over
      // both halves of every tile (the next pass cannot restart again)
      xmax[wave][lane & 15] = m_seen;
      __syncthreads();
      m_seen = fmaxf(m_seen, xmax[wave ^ 1][lane & 15]);
      __syncthreads();
      restart_flag = 0;
      issue_first_tiles();
    }

    // ---- finalise this piece ----
    // row sums and references of all 32 rows: lane l's output row is l % 32
    {
      float lw = l_run;
      lw += __shfl_xor(lw, 16);
      lw += __shfl_xor(lw, 32);
      xl[wave][lane & 15] = lw;
      xm[rh][lane & 15] = m_ref;  // both waves of a row pair hold the same reference
    }
    __syncthreads();
    const int orow = lane & 31;  // output row of this lane
    const int ohalf = orow >> 4, on = orow & 15;
    const float l_tot = xl[2 * ohalf][on] + xl[2 * ohalf + 1][on];
    const float m_row = xm[ohalf][on];
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float lse_v = l_tot > 0.f ? (m_row + fast_log2(l_tot)) * kLn2 : -INFINITY;
    const int g = lane >> 5;
    const int nrows = min(32, M);
    // acc[dt][v] is column 128 wave + 32 dt + 8 (v / 4) + 4 g + v % 4 of row orow
    float red;
    if (single && P.q_lat_lo != nullptr) {
      // first-order lse correction for the bf16 rounding of q_lat (see mla_decode_kernel)
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(P.q_lat_lo + (long long)b * M * kDLat), 0, M * kDLat * 2, kBufferWord3);
      const int base = min(orow, M - 1) * (kDLat * 2) + (128 * wave + 4 * g) * 2;
      float dot = 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const u32x2 q2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                         rl, base + (32 * dt + 8 * vq) * 2, 0, 0));
          const bf16x4 q4 = __builtin_bit_cast(bf16x4, q2);
#pragma unroll
          for (int e = 0; e < 4; ++e) dot += acc[dt][4 * vq + e] * (float)q4[e];
        }
      red = dot + __shfl_xor(dot, 32);
    } else {
      float amax = 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(acc[dt][v]));
      red = fmaxf(amax, __shfl_xor(amax, 32));
    }
    xred[wave][orow] = red;
    __syncthreads();
    const float r0 = xred[0][orow], r1 = xred[1][orow], r2 = xred[2][orow], r3 = xred[3][orow];
    // rows leave through LDS as whole 256-byte segments (this wave's columns);
    // the tile buffers are idle after the piece's last barrier
    MLA_LDS char* tw = lds + wave * (32 * 272);
    const int wr = orow * 272 + 8 * g;
    if (single) {
      if (P.q_lat_lo != nullptr && l_tot > 0.f) lse_v += P.scale * ((r0 + r1) + (r2 + r3)) * inv_l;
      const long long rbase = (long long)b * M;
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          P.o_lat + rbase * kDLat, 0, nrows * kDLat * 2, kBufferWord3);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[dt][4 * vq + e] * inv_l);
          *reinterpret_cast<MLA_LDS bf16x4*>(tw + wr + (32 * dt + 8 * vq) * 2) = w;
        }
#pragma unroll
      for (int k = 0; k < 8; ++k) {  // rows 4 k .. 4 k + 3, 256 bytes each
        const int r = 4 * k + (lane >> 4);
        const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(tw + r * 272 + (lane & 15) * 16);
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, r * (kDLat * 2) + wave * 256 + (lane & 15) * 16, 0, 0);
      }
      if (wave == 0) {
        const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(P.lse + rbase, 0, nrows * 4,
                                                                            kBufferWord3);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse_v), rl, orow * 4, 0, 0);
      }
    } else {
      const float amax = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
      const float mul = amax > 0.f ? 1.f / amax : 0.f;
      const long long pbase = (long long)split * M;
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          P.part_o + pbase * kDLat, 0, nrows * kDLat * 2, kBufferWord3);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          _Float16 w0 = (_Float16)(acc[dt][4 * vq + 0] * mul), w1 = (_Float16)(acc[dt][4 * vq + 1] * mul);
          _Float16 w2 = (_Float16)(acc[dt][4 * vq + 2] * mul), w3 = (_Float16)(acc[dt][4 * vq + 3] * mul);
          u32x2 w;
          w[0] = (unsigned)__builtin_bit_cast(unsigned short, w0) | ((unsigned)__builtin_bit_cast(unsigned short, w1) << 16);
          w[1] = (unsigned)__builtin_bit_cast(unsigned short, w2) | ((unsigned)__builtin_bit_cast(unsigned short, w3) << 16);
          *reinterpret_cast<MLA_LDS u32x2*>(tw + wr + (32 * dt + 8 * vq) * 2) = w;
        }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + (lane >> 4);
        const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(tw + r * 272 + (lane & 15) * 16);
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, r * (kDLat * 2) + wave * 256 + (lane & 15) * 16, 0, 0);
      }
      if (wave == 0) {
        const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(P.part_lse + pbase, 0, nrows * 4,
                                                                            kBufferWord3);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(P.part_scale + pbase, 0, nrows * 4,
                                                                            kBufferWord3);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, amax * inv_l), rs, orow * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse_v), rl, orow * 4, 0, 0);
      }
    }
  }
}

// Merge split partials: lse = ln sum_k exp(lse_k), o = sum_k exp(lse_k - lse) o_k,
// with o_k = scale_k * (fp16 row k).
// One workgroup per (sequence, 16 rows); 16 threads per row, each holding 32
// values as four 16-byte chunks (chunk t + 16 q of the row).
// Split-combine: one workgroup of four waves per (sequence, 4 R rows); a wave
// merges R rows, each spread over 64 / R lanes that hold R 16-byte chunks of
// it (chunk t + (64 / R) q of the row's 64), and keeps 16 / R pieces of every
// row in flight per group. R = 4 suits sequences cut into a few pieces
// (every lane has 16 loads in flight across its rows); R = 1 gives a
// sequence cut into many pieces 4x more waves, so each row's chain of
// dependent groups is 4x shorter.
// As in the decode kernels every branch is uniform over the wave: the piece
// count is a scalar load, a row without visible keys is weighed by arithmetic
// rather than skipped, and the lanes of a row all store its lse.
template <int R>
__global__ __launch_bounds__(256) void mla_combine_kernel(DecodeParams P) {
  constexpr int kLanesPerRow = 64 / R;
  constexpr int kGroup = 16 / R;  // pieces of every row whose loads are in flight together
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wrow0 = blockIdx.y * (4 * R) + wave_id_uniform() * R;  // first row of this wave
  // M is a multiple of 16, so a wave's R rows all lie inside it or all past it
  if (wrow0 >= P.M) return;
  const int row = wrow0 + lane / kLanesPerRow;
  const int t = lane % kLanesPerRow;
  const int ns0 = ldc(P.num_splits + b), n = ldc(P.num_splits + b + 1) - ns0;
  if (n == 1) return;
  const long long orow = (long long)b * P.M + row;
  u32x4* out = reinterpret_cast<u32x4*>(P.o_lat + orow * kDLat) + t;
  if (n == 0) {
#pragma unroll
    for (int q = 0; q < R; ++q) out[kLanesPerRow * q] = u32x4{};
    P.lse[orow] = -INFINITY;
    return;
  }
  // The lo residue of the row (first-order lse correction, see the decode
  // epilogue). With one row per wave it is loaded up front, so its latency
  // passes under the merge; with four, after it (its registers would cost a
  // wave per SIMD during the merge).
  u32x4 q8[R];
  const bool has_lo = P.q_lat_lo != nullptr;  // uniform (a test of a per-lane pointer would not be)
  const u32x4* qlo = reinterpret_cast<const u32x4*>(P.q_lat_lo + orow * kDLat) + t;
  if (R == 1 && has_lo) {
#pragma unroll
    for (int q = 0; q < R; ++q) q8[q] = qlo[kLanesPerRow * q];
  }
  // Streaming merge over the pieces, kGroup at a time with every load of a
  // group issued before any is used: running max m, weights exp(lse_k - m).
  float mx = -INFINITY, wsum = 0.f;
  float o[8 * R];
#pragma unroll
  for (int v = 0; v < 8 * R; ++v) o[v] = 0.f;
  for (int k0 = 0; k0 < n; k0 += kGroup) {
    float lk[kGroup], sk[kGroup];
    u32x4 src[kGroup][R];  // 8 fp16 values each
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      if (k0 + i < n) {  // uniform: the tail of the last group loads nothing and weighs zero
        const long long prow = (long long)(ns0 + k0 + i) * P.M + row;
        lk[i] = P.part_lse[prow];
        sk[i] = P.part_scale[prow];
        const u32x4* sp = reinterpret_cast<const u32x4*>(P.part_o + prow * kDLat) + t;
#pragma unroll
        for (int q = 0; q < R; ++q) src[i][q] = sp[kLanesPerRow * q];
      } else {
        lk[i] = -INFINITY;
        sk[i] = 0.f;
#pragma unroll
        for (int q = 0; q < R; ++q) src[i][q] = u32x4{};
      }
    }
    float m_new = mx;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) m_new = fmaxf(m_new, lk[i]);
    // While a row has seen nothing (m_new = -inf) every weight below is 0
    // and its sums stay 0, as if the group were skipped.
    const float m_s = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2((mx - m_s) * 1.4426950408889634f);  // 0 when mx = -inf
    wsum *= alpha;
#pragma unroll
    for (int v = 0; v < 8 * R; ++v) o[v] *= alpha;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float w = fast_exp2((lk[i] - m_s) * 1.4426950408889634f);  // 0 for the empty tail
      wsum += w;
      const float ws = w * sk[i];
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int h2 = 0; h2 < 4; ++h2) {
          const unsigned u = src[i][q][h2];
          o[8 * q + 2 * h2] += ws * (float)__builtin_bit_cast(_Float16, (unsigned short)(u & 0xffffu));
          o[8 * q + 2 * h2 + 1] += ws * (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> 16));
        }
    }
    mx = m_new;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float dot = 0.f;  // q_lo . o_lat
  if (R != 1 && has_lo) {
#pragma unroll
    for (int q = 0; q < R; ++q) q8[q] = qlo[kLanesPerRow * q];
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    bf16x8 w;
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = (__bf16)(o[8 * q + e] * inv);
    out[kLanesPerRow * q] = __builtin_bit_cast(u32x4, w);
    if (has_lo) {
      const bf16x8 qv = __builtin_bit_cast(bf16x8, q8[q]);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += o[8 * q + e] * inv * (float)qv[e];
    }
  }
#pragma unroll
  for (int m = kLanesPerRow / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);  // the row's lanes
  P.lse[orow] = wsum > 0.f ? mx + fast_log2(wsum) * kLn2 + P.scale * dot : -INFINITY;  // same value from each lane
}

// The page loader on its own: one workgroup per (page, sequence).
template <int NW>
__global__ __launch_bounds__(NW * 64) void mla_gather_kernel(DecodeParams P, const long long* row_offsets,
                                                            uint16_t* out) {
  __shared__ __attribute__((aligned(16))) char smem[kStageBytes];
  MLA_LDS char* lds = (MLA_LDS char*)(smem);
  const int page = blockIdx.x, b = blockIdx.y;
  const int L = P.seqlens[b];
  if (page * kPage >= L) return;
  const int lane = threadIdx.x & 63, wave = wave_id_uniform();
  TileLoad<NW> ld;
  const int pid = fetch_pid(P, b, page);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    ld.setup(P, page, half, L, pid, lds + half * kTileStageBytes, wave, lane);
#pragma unroll
    for (int i = 0; i < TileLoad<NW>::kInstr; ++i) ld.issue(i);
  }
  wait_vmem_all();
  __syncthreads();
  const int rows = min(kPage, L - page * kPage);
  u32x4* dst = reinterpret_cast<u32x4*>(out + (row_offsets[b] + (long long)page * kPage) * kDRow);
  for (int i = threadIdx.x; i < rows * (kRowBytes / 16); i += NW * 64) {
    const int r = i / (kRowBytes / 16), c = i - r * (kRowBytes / 16);
    dst[i] = *(const MLA_LDS u32x4*)(lds + lds_off(r, c));
  }
}

// Cache append: one wave per new row (72 chunks of 16 bytes; lane l copies
// chunks l and l + 64). Every check is uniform over the wave.
__global__ __launch_bounds__(64) void mla_append_kernel(const uint16_t* new_rows, uint16_t* kv,
                                                        long long num_pages, const int32_t* block_table,
                                                        int max_blocks, const int32_t* seqlens, int s_q) {
  const int b = blockIdx.x / s_q, j = blockIdx.x % s_q;
  const int lane = threadIdx.x;
  const int t = seqlens[b] - s_q + j;  // token index of this new row
  if (t < 0) {
    flag_error(MLA_DEVERR_SHORT_SEQ);
    return;
  }
  const int page = t / kPage;
  if (page >= max_blocks) {
    flag_error(MLA_DEVERR_SEQ_TOO_LONG);
    return;
  }
  const int pid = block_table[(long long)b * max_blocks + page];
  if (pid < 0 || pid >= num_pages) {
    flag_error(MLA_DEVERR_PAGE_ID);
    return;
  }
  const u32x4* src = reinterpret_cast<const u32x4*>(new_rows + ((long long)b * s_q + j) * kDRow);
  u32x4* dst = reinterpret_cast<u32x4*>(kv + ((long long)pid * kPage + (t % kPage)) * kDRow);
  constexpr int kChunks = kRowBytes / 16;  // 72
  const u32x4 v0 = src[lane];
  const u32x4 v1 = src[min(lane + 64, kChunks - 1)];
  dst[lane] = v0;
  if (lane + 64 < kChunks) dst[lane + 64] = v1;
}

// Scale exponent of a quantised row: the smallest e with amax <= 448 * 2^e,
// at least -126 (0 for an all-zero row), from the bits of amax: with
// amax = m * 2^E, m in [1, 2), e = E - 8, one more when m > 1.75.
__device__ __forceinline__ int fp8_scale_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const unsigned bits = __builtin_bit_cast(unsigned, amax);
  const int biased = (int)((bits >> 23) & 0xFF);
  if (biased == 0) return -126;  // below 2^-126 the floor applies
  const int e = biased - 127 - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return max(-126, e);
}

// One wave quantises one cache row: lane l takes latent values 8 l .. 8 l + 7;
// the wave's max |value| gives the scale 2^e; each value is divided by it
// (exact) and rounded to the nearest e4m3 code (ties to even; the values then
// lie within +-448). Lanes 0..15 copy the 64 bf16 key values, lane 0 writes
// the scale.
__device__ __forceinline__ void quantize_row_wave(const uint16_t* src, uint8_t* row, float* scale_slot, int lane) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(src + 8 * lane);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __builtin_bit_cast(float, v[i] << 16);
    x[2 * i + 1] = __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  const int e = fp8_scale_exponent(amax);
  u32x2 out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const unsigned lo =
        (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * w], -e), ldexpf(x[4 * w + 1], -e), 0, false) & 0xFFFFu;
    const unsigned hi =
        (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * w + 2], -e), ldexpf(x[4 * w + 3], -e), 0, false) & 0xFFFFu;
    out[w] = lo | (hi << 16);
  }
  *reinterpret_cast<u32x2*>(row + 8 * lane) = out;
  if (lane < 16) *reinterpret_cast<u32x2*>(row + kDLat + 8 * lane) = *reinterpret_cast<const u32x2*>(src + kDLat + 4 * lane);
  if (lane == 0) *scale_slot = ldexpf(1.0f, e);
}

// Whole-cache quantisation: one wave per row, 16 workgroups of 4 rows per page.
__global__ __launch_bounds__(256) void mla_quantize_pages_kernel(const uint16_t* kv, uint8_t* kv8) {
  const long long page = blockIdx.x / 16;
  const int row = (blockIdx.x % 16) * 4 + (threadIdx.x >> 6);
  uint8_t* dst = kv8 + page * kPageBytesF;
  quantize_row_wave(kv + (page * kPage + row) * kDRow, dst + row * kRowBytesF,
                    reinterpret_cast<float*>(dst + kScalesOffF) + row, threadIdx.x & 63);
}

// Quantise-on-append: one wave per new row, the checks of mla_append_kernel.
__global__ __launch_bounds__(64) void mla_append_fp8_kernel(const uint16_t* new_rows, uint8_t* kv8,
                                                            long long num_pages, const int32_t* block_table,
                                                            int max_blocks, const int32_t* seqlens, int s_q) {
  const int b = blockIdx.x / s_q, j = blockIdx.x % s_q;
  const int t = seqlens[b] - s_q + j;  // token index of this new row
  if (t < 0) {
    if (threadIdx.x == 0) flag_error(MLA_DEVERR_SHORT_SEQ);
    return;
  }
  const int page = t / kPage;
  if (page >= max_blocks) {
    if (threadIdx.x == 0) flag_error(MLA_DEVERR_SEQ_TOO_LONG);
    return;
  }
  const int pid = block_table[(long long)b * max_blocks + page];
  if (pid < 0 || pid >= num_pages) {
    if (threadIdx.x == 0) flag_error(MLA_DEVERR_PAGE_ID);
    return;
  }
  uint8_t* dst = kv8 + (long long)pid * kPageBytesF;
  quantize_row_wave(new_rows + ((long long)b * s_q + j) * kDRow, dst + (t % kPage) * kRowBytesF,
                    reinterpret_cast<float*>(dst + kScalesOffF) + (t % kPage), threadIdx.x);
}

}  // namespace mla

using namespace mla;

static int rows_per_wg_waves(int M) { return std::min(4, (M + 31) / 32); }

extern "C" int mla_num_slots(int b, int s_q, int h, int* num_slots) {
  if (!num_slots) return set_error(MLA_ERR_INVALID_ARG, "mla_num_slots: num_slots is NULL");
  if (int rc = check_shape("mla_num_slots", b, s_q, h)) return rc;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return set_error(MLA_ERR_HIP, "mla_num_slots: cannot query the device");
  const int M = s_q * h;
  const int nw = rows_per_wg_waves(M);
  const int R = (M + nw * 32 - 1) / (nw * 32);
  *num_slots = std::max(1, cus / R);
  return clear_error();
}

// Workspace: fp16 partial rows [splits, M, 512], then fp32 lse [splits, M]
// and fp32 row scales [splits, M], each region 256-byte aligned
// (splits = b + num_slots bounds the plan's pieces).
static size_t round256(size_t x) { return (x + 255) / 256 * 256; }
constexpr int kMaxSlots = 1 << 20;  // far beyond any useful grid

extern "C" size_t mla_workspace_bytes(int b, int s_q, int h, int num_slots) {
  // only shapes the decode accepts: the size below then cannot overflow
  if (b < 1 || b > MLA_MAX_BATCH || s_q < 1 || s_q > 8 || (h != 16 && h != 32 && h != 64 && h != 128) ||
      num_slots < 1 || num_slots > kMaxSlots)
    return 0;
  const size_t M = (size_t)s_q * h;
  const size_t splits = (size_t)b + num_slots;
  return round256(splits * M * kDLat * 2) + 2 * round256(splits * M * sizeof(float));
}

// Host checks shared by both decode entry points (everything but the workspace).
static int check_decode_args(const char* fn, const uint16_t* q_lat, const uint16_t* q_lat_lo, const uint16_t* q_pe,
                             const uint16_t* kv_cache, int64_t num_pages, const int32_t* block_table,
                             int max_blocks, const int32_t* cache_seqlens, int b, int s_q, int h,
                             float softmax_scale, const int32_t* tile_meta, const int32_t* num_splits,
                             int num_slots, uint16_t* o_lat, float* lse) {
  if (!q_lat || !q_pe || !kv_cache || !block_table || !cache_seqlens || !tile_meta || !num_splits || !o_lat ||
      !lse)
    return set_error(MLA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
  if (int rc = check_shape(fn, b, s_q, h)) return rc;
  if (b > MLA_MAX_BATCH) return set_error(MLA_ERR_INVALID_ARG, "%s: b must be <= %d (got %d)", fn, MLA_MAX_BATCH, b);
  if (num_pages < 1 || max_blocks < 1 || num_slots < 1)
    return set_error(MLA_ERR_INVALID_ARG, "%s: num_pages, max_blocks and num_slots must be >= 1", fn);
  if (num_slots > kMaxSlots) return set_error(MLA_ERR_INVALID_ARG, "%s: num_slots must be <= %d", fn, kMaxSlots);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return set_error(MLA_ERR_INVALID_ARG, "%s: softmax_scale must be positive and finite", fn);
  for (const void* p : {(const void*)q_lat, (const void*)q_pe, (const void*)kv_cache, (const void*)o_lat})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
      return set_error(MLA_ERR_INVALID_ARG, "%s: bf16 tensors must be 16-byte aligned", fn);
  if (q_lat_lo && reinterpret_cast<uintptr_t>(q_lat_lo) % 16 != 0)
    return set_error(MLA_ERR_INVALID_ARG, "%s: q_lat_lo must be 16-byte aligned", fn);
  return MLA_OK;
}

// Launches of one decode call (arguments already checked; `ws` holds at least
// mla_workspace_bytes(b, s_q, h, num_slots) bytes, 256-byte aligned).
static int decode_launch(const char* fn, const uint16_t* q_lat, const uint16_t* q_lat_lo, const uint16_t* q_pe,
                         const uint16_t* kv_cache, const uint8_t* kv8, int64_t num_pages,
                         const int32_t* block_table, int max_blocks,
                         const int32_t* cache_seqlens, int b, int s_q, int h, float softmax_scale, int causal,
                         const int32_t* tile_meta, const int32_t* num_splits, int num_slots, char* ws,
                         uint16_t* o_lat, float* lse, void* stream) {
  const int M = s_q * h;
  const int nw = rows_per_wg_waves(M);
  const int R = (M + nw * 32 - 1) / (nw * 32);
  const size_t M_ = (size_t)M, splits = (size_t)b + num_slots;
  DecodeParams P;
  P.q_lat = q_lat;
  P.q_lat_lo = q_lat_lo;
  P.q_pe = q_pe;
  P.kv = kv_cache;
  P.kv8 = kv8;
  P.block_table = block_table;
  P.seqlens = cache_seqlens;
  P.tile_meta = tile_meta;
  P.num_splits = num_splits;
  P.part_o = reinterpret_cast<uint16_t*>(ws);
  P.part_lse = reinterpret_cast<float*>(ws + round256(splits * M_ * kDLat * 2));
  P.part_scale = reinterpret_cast<float*>(ws + round256(splits * M_ * kDLat * 2) + round256(splits * M_ * 4));
  P.o_lat = o_lat;
  P.lse = lse;
  P.num_pages = num_pages;
  P.max_blocks = max_blocks;
  P.b = b;
  P.s_q = s_q;
  P.h = h;
  P.log2_h = __builtin_ctz((unsigned)h);
  P.M = M;
  P.n_rowblocks = R;
  P.num_slots = num_slots;
  P.causal = causal ? 1 : 0;
  P.scale = softmax_scale;
  P.scale_log2e = softmax_scale * 1.4426950408889634f;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int grid = R == 1 ? num_slots : ((num_slots + 7) / 8) * 8 * R;
  switch (nw) {
    case 1:
      if (kv8) hipLaunchKernelGGL(mla_decode_tsplit_kernel<true>, dim3(grid), dim3(256), 0, st, P);
      else hipLaunchKernelGGL(mla_decode_tsplit_kernel<false>, dim3(grid), dim3(256), 0, st, P);
      break;
    case 2: hipLaunchKernelGGL(mla_decode_kernel<2>, dim3(grid), dim3(128), 0, st, P); break;
    default: hipLaunchKernelGGL(mla_decode_kernel<4>, dim3(grid), dim3(256), 0, st, P); break;
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: decode launch failed: %s", fn, hipGetErrorString(e));
  // The plan cuts the batch into at most b + num_slots - 1 pieces. When that
  // averages more than four per sequence, one row per combine wave (R = 1);
  // otherwise four (R = 4).
  if ((long long)b + num_slots - 1 > 4LL * b)
    hipLaunchKernelGGL(mla_combine_kernel<1>, dim3(b, (M + 3) / 4), dim3(256), 0, st, P);
  else
    hipLaunchKernelGGL(mla_combine_kernel<4>, dim3(b, (M + 15) / 16), dim3(256), 0, st, P);
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: combine launch failed: %s", fn, hipGetErrorString(e));
  return clear_error();
}

extern "C" int mla_decode_paged(const uint16_t* q_lat, const uint16_t* q_lat_lo, const uint16_t* q_pe,
                                const uint16_t* kv_cache, int64_t num_pages, const int32_t* block_table,
                                int max_blocks, const int32_t* cache_seqlens, int b, int s_q, int h,
                                float softmax_scale, int causal, const int32_t* tile_meta,
                                const int32_t* num_splits, int num_slots, void* workspace,
                                size_t workspace_bytes, uint16_t* o_lat, float* lse, void* stream) {
  const char* fn = "mla_decode_paged";
  if (!workspace) return set_error(MLA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
  if (int rc = check_decode_args(fn, q_lat, q_lat_lo, q_pe, kv_cache, num_pages, block_table, max_blocks,
                                 cache_seqlens, b, s_q, h, softmax_scale, tile_meta, num_splits, num_slots, o_lat,
                                 lse))
    return rc;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return set_error(MLA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  const size_t need = mla_workspace_bytes(b, s_q, h, num_slots);
  if (workspace_bytes < need)
    return set_error(MLA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, need);
  return decode_launch(fn, q_lat, q_lat_lo, q_pe, kv_cache, nullptr, num_pages, block_table, max_blocks,
                       cache_seqlens, b, s_q, h, softmax_scale, causal, tile_meta, num_splits, num_slots,
                       static_cast<char*>(workspace), o_lat, lse, stream);
}

// Scratch of mla_decode_paged_noalloc: one fixed array per GPU, in the
// library's device code object, in place of the caller's workspace. In host
// code `scratch` names a host-side stand-in, not device memory: the device
// address comes from hipGetSymbolAddress, once per device (with that device
// current), and only that address is ever passed to a kernel.
static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch` per device id (null until resolved)
}  // namespace

static int scratch_for_current_device(const char* fn, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return set_error(MLA_ERR_HIP, "%s: cannot query the current device", fn);
  if (dev >= kMaxDevices)
    return set_error(MLA_ERR_UNSUPPORTED, "%s: device %d is beyond the %d devices this call supports", fn, dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_error(MLA_ERR_HIP, "%s: cannot resolve the scratch array on device %d: %s", fn, dev,
                       hipGetErrorString(e));
    if (reinterpret_cast<uintptr_t>(p) % 256 != 0)
      return set_error(MLA_ERR_HIP, "%s: the scratch array on device %d is not 256-byte aligned", fn, dev);
    g_scratch_dev[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_dev[dev]);
  return MLA_OK;
}

extern "C" int mla_decode_paged_noalloc(const uint16_t* q_lat, const uint16_t* q_lat_lo, const uint16_t* q_pe,
                                        const uint16_t* kv_cache, int64_t num_pages, const int32_t* block_table,
                                        int max_blocks, const int32_t* cache_seqlens, int b, int s_q, int h,
                                        float softmax_scale, int causal, const int32_t* tile_meta,
                                        const int32_t* num_splits, int num_slots, uint16_t* o_lat, float* lse,
                                        void* stream) {
  const char* fn = "mla_decode_paged_noalloc";
  if (int rc = check_decode_args(fn, q_lat, q_lat_lo, q_pe, kv_cache, num_pages, block_table, max_blocks,
                                 cache_seqlens, b, s_q, h, softmax_scale, tile_meta, num_splits, num_slots, o_lat,
                                 lse))
    return rc;
  const size_t need = mla_workspace_bytes(b, s_q, h, num_slots);
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
    return set_error(MLA_ERR_WORKSPACE,
                     "%s: this shape needs %zu bytes of split partials (b=%d, s_q=%d, h=%d, num_slots=%d), more "
                     "than the %zu-byte built-in scratch; use mla_decode_paged with a workspace",
                     fn, need, b, s_q, h, num_slots, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  char* ws = nullptr;
  if (int rc = scratch_for_current_device(fn, &ws)) return rc;
  return decode_launch(fn, q_lat, q_lat_lo, q_pe, kv_cache, nullptr, num_pages, block_table, max_blocks,
                       cache_seqlens, b, s_q, h, softmax_scale, causal, tile_meta, num_splits, num_slots, ws, o_lat,
                       lse, stream);
}

extern "C" int mla_gather_pages(const uint16_t* kv_cache, int64_t num_pages, const int32_t* block_table,
                                int max_blocks, const int32_t* cache_seqlens, int b,
                                const int64_t* row_offsets, uint16_t* out, void* stream) {
  const char* fn = "mla_gather_pages";
  if (!kv_cache || !block_table || !cache_seqlens || !row_offsets || !out)
    return set_error(MLA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
  if (b < 1 || num_pages < 1 || max_blocks < 1)
    return set_error(MLA_ERR_INVALID_ARG, "%s: b, num_pages and max_blocks must be >= 1", fn);
  if (reinterpret_cast<uintptr_t>(kv_cache) % 16 || reinterpret_cast<uintptr_t>(out) % 16)
    return set_error(MLA_ERR_INVALID_ARG, "%s: kv_cache and out must be 16-byte aligned", fn);
  DecodeParams P{};
  P.kv = kv_cache;
  P.block_table = block_table;
  P.seqlens = cache_seqlens;
  P.num_pages = num_pages;
  P.max_blocks = max_blocks;
  P.b = b;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // one wave and four waves take different shares of the same load pattern
  hipLaunchKernelGGL(mla_gather_kernel<4>, dim3(max_blocks, b), dim3(256), 0, st, P,
                     reinterpret_cast<const long long*>(row_offsets), out);
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return clear_error();
}

extern "C" int mla_append_kv(const uint16_t* new_rows, uint16_t* kv_cache, int64_t num_pages,
                             const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens, int b,
                             int s_q, void* stream) {
  const char* fn = "mla_append_kv";
  if (!new_rows || !kv_cache || !block_table || !cache_seqlens)
    return set_error(MLA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
  if (b < 1) return set_error(MLA_ERR_INVALID_ARG, "%s: b must be >= 1 (got %d)", fn, b);
  if (s_q < 1 || s_q > 8) return set_error(MLA_ERR_INVALID_ARG, "%s: s_q must be in [1, 8] (got %d)", fn, s_q);
  if (num_pages < 1 || max_blocks < 1)
    return set_error(MLA_ERR_INVALID_ARG, "%s: num_pages and max_blocks must be >= 1", fn);
  if (reinterpret_cast<uintptr_t>(new_rows) % 16 || reinterpret_cast<uintptr_t>(kv_cache) % 16)
    return set_error(MLA_ERR_INVALID_ARG, "%s: new_rows and kv_cache must be 16-byte aligned", fn);
  hipLaunchKernelGGL(mla_append_kernel, dim3(b * s_q), dim3(64), 0, static_cast<hipStream_t>(stream), new_rows,
                     kv_cache, (long long)num_pages, block_table, max_blocks, cache_seqlens, s_q);
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return clear_error();
}

extern "C" int mla_take_device_error(int* bits) {
  if (!bits) return set_error(MLA_ERR_INVALID_ARG, "mla_take_device_error: bits is NULL");
  int v = 0, zero = 0;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_device_error), sizeof(int), 0, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(g_device_error), &zero, sizeof(int), 0, hipMemcpyHostToDevice) != hipSuccess)
    return set_error(MLA_ERR_HIP, "mla_take_device_error: cannot read the device error word");
  *bits = v;
  return clear_error();
}

extern "C" int mla_decode_paged_fp8(const uint16_t* q_lat, const uint16_t* q_lat_lo, const uint16_t* q_pe,
                                    const uint8_t* kv_fp8, int64_t num_pages, const int32_t* block_table,
                                    int max_blocks, const int32_t* cache_seqlens, int b, int s_q, int h,
                                    float softmax_scale, int causal, const int32_t* tile_meta,
                                    const int32_t* num_splits, int num_slots, void* workspace,
                                    size_t workspace_bytes, uint16_t* o_lat, float* lse, void* stream) {
  const char* fn = "mla_decode_paged_fp8";
  if (!workspace) return set_error(MLA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
  if (int rc = check_decode_args(fn, q_lat, q_lat_lo, q_pe, reinterpret_cast<const uint16_t*>(kv_fp8), num_pages,
                                 block_table, max_blocks, cache_seqlens, b, s_q, h, softmax_scale, tile_meta,
                                 num_splits, num_slots, o_lat, lse))
    return rc;
  if (s_q * h > 32)
    return set_error(MLA_ERR_UNSUPPORTED, "%s: built for at most 32 query rows per sequence (s_q * h = %d)", fn,
                     s_q * h);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return set_error(MLA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  const size_t need = mla_workspace_bytes(b, s_q, h, num_slots);
  if (workspace_bytes < need)
    return set_error(MLA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, need);
  return decode_launch(fn, q_lat, q_lat_lo, q_pe, nullptr, kv_fp8, num_pages, block_table, max_blocks, cache_seqlens,
                       b, s_q, h, softmax_scale, causal, tile_meta, num_splits, num_slots,
                       static_cast<char*>(workspace), o_lat, lse, stream);
}

extern "C" int mla_quantize_pages(const uint16_t* kv_cache, int64_t num_pages, uint8_t* kv_fp8, void* stream) {
  const char* fn = "mla_quantize_pages";
  if (!kv_cache || !kv_fp8) return set_error(MLA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
  if (num_pages < 1 || num_pages > (1LL << 26))
    return set_error(MLA_ERR_INVALID_ARG, "%s: num_pages must be in [1, 2^26] (got %lld)", fn, (long long)num_pages);
  if (reinterpret_cast<uintptr_t>(kv_cache) % 16 || reinterpret_cast<uintptr_t>(kv_fp8) % 16)
    return set_error(MLA_ERR_INVALID_ARG, "%s: kv_cache and kv_fp8 must be 16-byte aligned", fn);
  hipLaunchKernelGGL(mla_quantize_pages_kernel, dim3((unsigned)(num_pages * 16)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), kv_cache, kv_fp8);
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return clear_error();
}

extern "C" int mla_append_kv_fp8(const uint16_t* new_rows, uint8_t* kv_fp8, int64_t num_pages,
                                 const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens, int b,
                                 int s_q, void* stream) {
  const char* fn = "mla_append_kv_fp8";
  if (!new_rows || !kv_fp8 || !block_table || !cache_seqlens)
    return set_error(MLA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
  if (b < 1) return set_error(MLA_ERR_INVALID_ARG, "%s: b must be >= 1 (got %d)", fn, b);
  if (s_q < 1 || s_q > 8) return set_error(MLA_ERR_INVALID_ARG, "%s: s_q must be in [1, 8] (got %d)", fn, s_q);
  if (num_pages < 1 || max_blocks < 1)
    return set_error(MLA_ERR_INVALID_ARG, "%s: num_pages and max_blocks must be >= 1", fn);
  if (reinterpret_cast<uintptr_t>(new_rows) % 16 || reinterpret_cast<uintptr_t>(kv_fp8) % 16)
    return set_error(MLA_ERR_INVALID_ARG, "%s: new_rows and kv_fp8 must be 16-byte aligned", fn);
  hipLaunchKernelGGL(mla_append_fp8_kernel, dim3(b * s_q), dim3(64), 0, static_cast<hipStream_t>(stream), new_rows,
                     kv_fp8, (long long)num_pages, block_table, max_blocks, cache_seqlens, s_q);
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return set_error(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return clear_error();
}
