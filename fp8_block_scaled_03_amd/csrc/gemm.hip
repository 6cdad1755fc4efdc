// E4M3 GEMM with 32x32 block scales for gfx950 (MI355X).
//
// C[i,j] = sum_kb sa[i/32,kb] * sb[kb,j/32] * sum_{k in kb} A[i,k] B[k,j]
// (DeepGEMM write-up on hncyxsy.com, sections 2.2-2.3), every element computed
// with the one recipe in common.hpp; K is never split across accumulators and
// K-blocks are promoted in ascending order, so an element's bits do not depend
// on M, on its position in the tile or on which kernel ran ("AI Infra 进阶：
// 如何让大模型输出确定的结果", part 一 sections 6-7: batch invariance needs a
// fixed reduction order, no M-dependent split-K).
//
// Kernels:
//  * tile kernel (large M, and the grouped variant): a 512-thread workgroup owns
//    a 256x256 C tile; eight waves in a 4(M) x 2(N) grid own 64x128 each
//    (4 x 8 MFMA sub-tiles of 16x16).  Per 32-deep K-block the workgroup
//    loads 8 KB of A and 8 KB of B (16 bytes per thread each, coalesced, two
//    iterations ahead in two register sets), decodes E4M3 -> bf16 once, and
//    stores the bf16 tiles into a four-stage LDS ring (one barrier per two
//    K-blocks) with an XOR swizzle so that the fragment reads are free of
//    bank conflicts (DeepGEMM write-up, section 3.1, makes the same point for
//    shared memory; section 3.3 for overlapping the next tile's loads with
//    compute).  A fragments are read K-contiguous with ds_read_b128; B is
//    N-contiguous in memory, so its fragments come from the LDS transpose read
//    ds_read_b64_tr_b16 (a K-major weight is staged like A instead).  Waves
//    whose 64-row band lies wholly past the problem's rows only stage and meet
//    the barriers; a tile with at most 128 rows runs the light body (eight
//    64 x 64 wave tiles over 128 x 256).
//  * small-M kernels (M <= 64, decode): a workgroup owns a slice of 32, 64 or
//    128 columns of C for all rows and all of K and streams its slice of the
//    weight once, eight K-blocks per round, with direct global->LDS loads into
//    a ring several rounds deep.  Waves own whole 16x16 output sub-tiles and
//    run their promotion chains in ascending K-block order (with 17-32 rows
//    on 128-column slices A is decoded once per workgroup into a shared bf16
//    area); for one-tile slices of a K-major weight the split kernel instead
//    forms each K-block's partials on a different wave and promotes them in
//    order one round later.
#include "common.hpp"

#include <type_traits>

namespace fp8bs {

// ------------------------------------------------------------------------------------
// tile kernel
// ------------------------------------------------------------------------------------
constexpr int TBM = 256, TBN = 256, TTHREADS = 512;
constexpr int A_STAGE_BYTES = TBM * 32 * 2;  // 16 KB bf16
constexpr int B_STAGE_BYTES = 32 * TBN * 2 + 512;  // 16 KB bf16 + row-group shifts
constexpr int STAGE_BYTES = A_STAGE_BYTES + B_STAGE_BYTES;
constexpr int TILE_STAGES = 4;
// Scale products s = sa * sb are formed once per workgroup in windows of SCW
// K-blocks (double-buffered in LDS): per K-block 8 row-blocks x 8 column-blocks.
constexpr int SCW = 32;
constexpr int SC_WINDOW_BYTES = SCW * 8 * 8 * 4;  // 8 KB
// Per-token-group activation scales: the window holds raw sa of the tile's 256
// rows and raw sb of its 8 column blocks for SCWT K-blocks.
constexpr int SCWT = 8;
constexpr int TG_WINDOW_FLOATS = SCWT * (256 + 8);
constexpr int TG_WINDOW_BYTES = TG_WINDOW_FLOATS * 4;  // 8.25 KB
constexpr int TILE_SC_BYTES = 2 * (SC_WINDOW_BYTES > TG_WINDOW_BYTES ? SC_WINDOW_BYTES : TG_WINDOW_BYTES);
constexpr int TILE_LDS_BYTES = TILE_STAGES * STAGE_BYTES + TILE_SC_BYTES;  // 146.5 KB
static_assert(TILE_LDS_BYTES <= 160 * 1024, "LDS budget");

// A tile in LDS: [256 rows][4 chunks of 8 bf16]; chunk c of row r lives at
// position c ^ ((r >> 1) & 3).
__device__ __forceinline__ int a_lds_off(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4); }
// B tile in LDS: [32 k][16 chunks of 16 bf16 (32 bytes)]; chunk j of row k lives at
// position j ^ (k & 3), and each group of 8 rows is shifted by a further 128
// bytes: one transposed read touches rows k and k+8 together, and the shift
// puts them in different banks.
__device__ __forceinline__ int b_lds_off(int k, int chunk) {
  return k * 512 + (k >> 3) * 128 + ((chunk ^ (k & 3)) << 5);
}

// A zero in device memory: the token-group scale window loads it (with a direct
// global->LDS load, like every other entry) as sb past the last K-block.
__device__ const float kZeroScale = 0.0f;

struct TileArgs {
  const uint8_t* a;   // rows of this problem start here (global row index 0)
  const float* sa;    // [ceil(M/32), KB]
  const uint8_t* b;   // [K, N], or [N, K] when the weight is K-major
  const float* sb;    // [KB, NB], or [NB, KB] when the weight is K-major
  uint16_t* c;        // [.., N]
  int64_t N, K;
  int64_t row0;       // first row of the tile
  int64_t row_end;    // rows >= row_end are not part of this problem
  int64_t col0;       // first column of the tile
  int64_t sa_rows;    // number of scale rows (for clamping)
};

// BT: the weight is K-major (B^T, [N, K]); its rows are staged and read exactly
// like rows of A (K-contiguous, no transposed LDS reads), and its scale grid is
// [NB, KB].
// TG: A carries per-token-group scales sa [M, KB] (one per row and K-block).
// The MFMA then takes the B fragment as its first operand and the A fragment
// as its second, so a lane's four outputs share one row of C (and one 32-column
// block): the scale sa[row, kb] * sb[kb, cb] is one value per lane per
// sub-tile.  Every kernel that takes token-group scales forms its partials
// this way.
//
// LIGHT: a tile with at most 128 rows of the problem.  The staging, the LDS
// layout and the scale window are the full tile's, but the eight waves cover
// the first 128 rows only: two row bands of 64 and four column bands of 64
// (a 64 x 64 wave tile).  With 65-128 rows every SIMD runs two busy waves;
// with at most 64, one.  Each output element is formed by the same MFMAs and
// promotions in the same order as in the full tile.
template <bool BT, bool TG, bool LIGHT = false>
__device__ __forceinline__ void tile_body(const TileArgs& p, unsigned char* smem) {
  static_assert(!(LIGHT && TG), "the light tile is used with 32x32 scales only");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = wave_id_uniform();
  // Waves are dealt to the four SIMDs round-robin (wave w on SIMD w % 4), so
  // row band wm = w >> 1 gives every SIMD one wave in the tile's upper half
  // and one in its lower half: in a tile whose last rows lie past the
  // problem, the waves of bands with no rows skip their MFMAs and promotions
  // and every SIMD keeps one busy wave.  In a light tile, waves w and w + 4
  // (one SIMD) take the two row bands of column band w & 3.
  constexpr int JN = LIGHT ? 4 : 8;           // 16-column sub-tiles per wave
  constexpr int WN_T = JN * 16;               // columns per wave
  constexpr int NQ = 4 * JN;                  // MFMAs per wave and K-block
  const int wm = LIGHT ? (w >> 2) : (w >> 1);
  const int wn = LIGHT ? (w & 3) : (w & 1);
  const int64_t K = p.K, N = p.N;
  const int KB = (int)(K >> 5);
  const int NB = (int)(N >> 5);
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  lds_u8* const sA = (lds_u8*)smem;                            // 3 A stages
  lds_u8* const sB = sA + TILE_STAGES * A_STAGE_BYTES;         // 3 B stages

  // ---- global -> register staging assignment
  const int a_row = t >> 1, a_half = t & 1;           // 16 E4M3 of A row a_row
  const int64_t ga_row = p.row0 + a_row;
  const bool a_ok = ga_row < p.row_end;
  const uint8_t* a_src = p.a + (a_ok ? ga_row : 0) * K + a_half * 16;
  // B [K, N]: 16 E4M3 of K-row t>>4, 16-column chunk t&15.  B^T [N, K]: like A,
  // 16 E4M3 of weight row (column of C) col0 + (t>>1), half t&1 of the K-block.
  bool b_ok;
  const uint8_t* b_src;
  lds_u8* st_b;
  lds_u8* st_b1;
  if constexpr (BT) {
    const int64_t gn = p.col0 + (t >> 1);
    b_ok = gn < N;
    b_src = p.b + (b_ok ? gn : 0) * K + (t & 1) * 16;
    st_b = sB + a_lds_off(t >> 1, 2 * (t & 1));
    st_b1 = sB + a_lds_off(t >> 1, 2 * (t & 1) + 1);
  } else {
    const int b_row = t >> 4, b_chunk = t & 15;
    b_ok = (p.col0 + b_chunk * 16) < N;
    b_src = p.b + (int64_t)b_row * N + (b_ok ? p.col0 + b_chunk * 16 : 0);
    st_b = sB + b_lds_off(b_row, b_chunk);
    st_b1 = st_b + 16;
  }
  // LDS store addresses (stage 0); other stages add a compile-time offset
  lds_u8* const st_a0 = sA + a_lds_off(a_row, 2 * a_half);
  lds_u8* const st_a1 = sA + a_lds_off(a_row, 2 * a_half + 1);

  // Rows of A past the problem and columns of B past N load a clamped, valid
  // address instead of zeros: they feed only outputs that are never stored.
  // Unconditional loads let the compiler count them exactly, so the wait before
  // staging covers only the K-block being staged, not the one loaded after it.
  auto load_a_only = [&](int kb, uint4& ra) __attribute__((always_inline)) {
    ra = *reinterpret_cast<const uint4*>(a_src + (int64_t)kb * 32);
  };
  auto load_b_only = [&](int kb, uint4& rb) __attribute__((always_inline)) {
    const int64_t boff = BT ? (int64_t)kb * 32 : (int64_t)kb * 32 * N;
    rb = *reinterpret_cast<const uint4*>(b_src + boff);
  };
  auto load_stage = [&](int kb, uint4& ra, uint4& rb) __attribute__((always_inline)) {
    load_a_only(kb, ra);
    load_b_only(kb, rb);
  };
  // `st` is the stage index (wave-uniform, 0..2)
  auto store_stage = [&](int st, uint4 ra, uint4 rb) __attribute__((always_inline)) {
    uint4 a0, a1, b0, b1;
    e4m3x16_to_bf16x16(ra, a0, a1);
    e4m3x16_to_bf16x16(rb, b0, b1);
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4u lds_v4u;
    const int soa = st * A_STAGE_BYTES, sob = st * B_STAGE_BYTES;
    *(lds_v4u*)(st_a0 + soa) = v4u{a0.x, a0.y, a0.z, a0.w};
    *(lds_v4u*)(st_a1 + soa) = v4u{a1.x, a1.y, a1.z, a1.w};
    *(lds_v4u*)(st_b + sob) = v4u{b0.x, b0.y, b0.z, b0.w};
    *(lds_v4u*)(st_b1 + sob) = v4u{b1.x, b1.y, b1.z, b1.w};
  };
  // One quarter of store_stage: 8 E4M3 bytes (half of ra or rb) -> 8 bf16 ->
  // one 16-byte LDS store.  piece 0/1: the low/high half of ra (A), 2/3: of rb.
  auto store_piece = [&](int st, int piece, uint4 ra, uint4 rb) __attribute__((always_inline)) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4u lds_v4u;
    const uint4 src = piece < 2 ? ra : rb;
    const uint32_t w0 = (piece & 1) ? src.z : src.x, w1 = (piece & 1) ? src.w : src.y;
    const v2i x = e4m3x4_to_bf16x4(w0), y = e4m3x4_to_bf16x4(w1);
    lds_u8* dst = piece == 0 ? st_a0 + st * A_STAGE_BYTES : piece == 1 ? st_a1 + st * A_STAGE_BYTES
                : piece == 2 ? st_b + st * B_STAGE_BYTES : st_b1 + st * B_STAGE_BYTES;
    *(lds_v4u*)dst = v4u{(unsigned)x[0], (unsigned)x[1], (unsigned)y[0], (unsigned)y[1]};
  };

  // ---- fragment read addresses.  A: row wm*64 + i*16 + (lane&15), chunk lane>>4;
  // the swizzle term depends only on the lane, so sub-tile i is +1024 bytes.
  const int fr_lo = lane & 15, fr_kc = lane >> 4;
  const lds_u8* const rd_a = sA + a_lds_off(wm * 64 + fr_lo, fr_kc);
  // B (transposed reads): lane (g, r, c) = (lane>>4, (lane>>2)&3, lane&3) reads row
  // k = 8g + 4h + r, 32-byte chunk J = wn*JN + j at position J ^ r, byte 8c.
  // J ^ r = wn*JN + 4*(j>>2) + ((j&3) ^ r): four lane-dependent bases, the rest
  // (h, j>>2, the stage) compile-time offsets.
  const int tr_g = lane >> 4, tr_r = (lane >> 2) & 3, tr_c = lane & 3;
  const lds_u8* rd_b[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
    rd_b[jj] = sB + b_lds_off(8 * tr_g + tr_r, wn * JN + jj) + tr_c * 8;
  auto read_a = [&](int st, int i) __attribute__((always_inline)) -> v8bf {
    typedef __attribute__((address_space(3))) const v8bf lds_v8bf;
    return *(lds_v8bf*)(rd_a + st * A_STAGE_BYTES + i * 1024);
  };
  // B^T: weight row wn*WN_T + j*16 + (lane&15), chunk lane>>4, read like A
  const lds_u8* const rd_bt = sB + a_lds_off(wn * WN_T + fr_lo, fr_kc);
  auto read_b = [&](int st, int j) __attribute__((always_inline)) -> v8bf {
    if constexpr (BT) {
      typedef __attribute__((address_space(3))) const v8bf lds_v8bf;
      return *(lds_v8bf*)(rd_bt + st * B_STAGE_BYTES + j * 1024);
    }
    const lds_u8* base = rd_b[j & 3] + st * B_STAGE_BYTES + (j >> 2) * 128;
    v4s h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base));
    v4s h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base + 4 * 512));
    v2i x0 = __builtin_bit_cast(v2i, h0), x1 = __builtin_bit_cast(v2i, h1);
    return __builtin_bit_cast(v8bf, v4i{x0[0], x0[1], x1[0], x1[1]});
  };

  // ---- scale products.  Window buffer [2][SCW K-blocks][8 row-blocks][8 col-blocks]
  // of s = sa * sb (one fp32 multiply, the same rounding every kernel uses).
  // Thread t forms (row-block, col-block) = ((t>>3)&7, t&7) for K-blocks
  // t>>6, t>>6 + 8, ...; rows or columns past the operand are clamped to a
  // valid block (never stored).
  float* const sc_lds = reinterpret_cast<float*>(smem + TILE_STAGES * STAGE_BYTES);  // after A and B stages
  const int64_t rb_tile = p.row0 >> 5, cb_tile = p.col0 >> 5;
  const int w_rb = (t >> 3) & 7, w_cb = t & 7, w_k0 = t >> 6;
  int64_t sa_row = rb_tile + w_rb;
  sa_row = sa_row < p.sa_rows ? sa_row : p.sa_rows - 1;
  int64_t sb_col = cb_tile + w_cb;
  sb_col = sb_col < NB ? sb_col : NB - 1;
  const float* const sa_src = p.sa + sa_row * KB;
  const float* const sb_src = BT ? p.sb + sb_col * KB : p.sb + sb_col;
  const int64_t sb_kstride = BT ? 1 : NB;
  auto load_scale_window = [&](int win) __attribute__((always_inline)) {
    float* dst = sc_lds + (win & 1) * (SCW * 64);
    float va[SCW / 8], vb[SCW / 8];
#pragma unroll
    for (int i = 0; i < SCW / 8; ++i) {
      int kk = win * SCW + w_k0 + 8 * i;
      kk = kk < KB ? kk : KB - 1;  // past the end: read any valid block, store 0
      va[i] = sa_src[kk];
      vb[i] = sb_src[(int64_t)kk * sb_kstride];
    }
#pragma unroll
    for (int i = 0; i < SCW / 8; ++i)
      dst[(w_k0 + 8 * i) * 64 + w_rb * 8 + w_cb] = win * SCW + w_k0 + 8 * i < KB ? va[i] * vb[i] : 0.0f;
  };
  // this wave's blocks: rows wm*64.. (row-blocks 2wm, 2wm+1), cols wn*WN_T..
  // (col-blocks CBW*wn .. CBW*wn + CBW-1)
  typedef float v4f_t __attribute__((ext_vector_type(4)));
  typedef float v2f_t __attribute__((ext_vector_type(2)));
  constexpr int CBW = JN / 2;
  auto read_scales = [&](int kb, float (&sc)[2][CBW]) __attribute__((always_inline)) {
    const float* w0 = sc_lds + ((kb / SCW) & 1) * (SCW * 64) + (kb % SCW) * 64 + (2 * wm) * 8 + CBW * wn;
    if constexpr (CBW == 4) {
      const v4f_t r0 = *reinterpret_cast<const v4f_t*>(w0);
      const v4f_t r1 = *reinterpret_cast<const v4f_t*>(w0 + 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[0][j] = r0[j];
        sc[1][j] = r1[j];
      }
    } else {
      const v2f_t r0 = *reinterpret_cast<const v2f_t*>(w0);
      const v2f_t r1 = *reinterpret_cast<const v2f_t*>(w0 + 8);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        sc[0][j] = r0[j];
        sc[1][j] = r1[j];
      }
    }
  };

  // token-group scales: window [2][SCWT][256 rows + 8 col-blocks] of raw sa / sb.
  // Row r = wm*64 + 16*ui + lo of the tile sits at [kk][wm][lo][ui], so a lane
  // reads the sa of its four rows (lo = lane & 15, ui = 0..3) with one 16-byte
  // read.
  // Filled with direct global->LDS dword loads (no registers): dword d of the
  // window is loaded by lane d % 64 of load d / 64, and waited for with an
  // explicit vmcnt count before the barrier that ends the iteration (only
  // that iteration's two operand loads may still be in flight).
  const uint32_t sc_lds_addr = (uint32_t)(uintptr_t)((lds_u8*)sc_lds);
  auto load_tg_window = [&](int win) __attribute__((always_inline)) {
    const uint32_t dst = sc_lds_addr + (win & 1) * TG_WINDOW_BYTES;
    for (int i = w; i < TG_WINDOW_FLOATS / 64; i += TTHREADS / 64) {
      const int pos = i * 64 + lane;
      const float* src;
      if (pos < SCWT * 256) {
        const int kk = pos >> 8, within = pos & 255;
        const int rr = (within >> 6) * 64 + (within & 3) * 16 + ((within >> 2) & 15);
        int kb = win * SCWT + kk;
        kb = kb < KB ? kb : KB - 1;
        int64_t row = p.row0 + rr;
        row = row < p.row_end ? row : p.row_end - 1;
        src = p.sa + row * KB + kb;
      } else {
        const int j = pos - SCWT * 256, kk = j >> 3, cbl = j & 7;
        int kb = win * SCWT + kk;
        const bool past = kb >= KB;  // past the last K-block: sb = 0
        kb = past ? KB - 1 : kb;
        int64_t cb = cb_tile + cbl;
        cb = cb < NB ? cb : NB - 1;
        src = past ? &kZeroScale : BT ? p.sb + cb * KB + kb : p.sb + (int64_t)kb * NB + cb;
      }
      dma4(src, dst + i * 256);
    }
  };
  // sa of the lane's four rows and sb of the wave's four column blocks, both
  // in VGPRs (moving sb to SGPRs with v_readfirstlane measured 1.7% slower)
  auto read_tg_scales = [&](int kb, v4f_t& sa4, float (&sbs)[4]) __attribute__((always_inline)) {
    const float* w0 = sc_lds + ((kb / SCWT) & 1) * TG_WINDOW_FLOATS;
    const int kk = kb % SCWT;
    sa4 = *reinterpret_cast<const v4f_t*>(w0 + kk * 256 + wm * 64 + (lane & 15) * 4);
    const v4f_t sb4 = *reinterpret_cast<const v4f_t*>(w0 + SCWT * 256 + kk * 8 + 4 * wn);
#pragma unroll
    for (int j = 0; j < 4; ++j) sbs[j] = sb4[j];
  };

  v4f acc[4][JN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- prologue: K-blocks 0-2 staged in LDS, K-blocks 3 and 4 in the two
  // register sets, K-block 0's fragments in registers
  // K = 0: no operand or scale is touched (the caller may pass null pointers);
  // the accumulators stay zero.
  if (KB > 0) {
    if constexpr (TG) {
      load_tg_window(0);
      wait_vmcnt<0>();
    } else {
      load_scale_window(0);
    }
  }
  uint4 ra = make_uint4(0, 0, 0, 0), rb = make_uint4(0, 0, 0, 0);
  // stages 0-2 hold K-blocks 0-2, clamped to the last one: the empty K-blocks
  // that pad KB to a multiple of four multiply finite codes
  if (KB > 0) { load_stage(0, ra, rb); store_stage(0, ra, rb); }
  if (KB > 0) { load_stage(KB > 1 ? 1 : KB - 1, ra, rb); store_stage(1, ra, rb); }
  if (KB > 0) { load_stage(KB > 2 ? 2 : KB - 1, ra, rb); store_stage(2, ra, rb); }
  // The two register sets are loaded in the order the loop reloads them (A then
  // B of the first set, then the second): the loop entry then matches the
  // steady state, and the compiler can count the loads in flight exactly.
  uint4 ra2 = make_uint4(0, 0, 0, 0), rb2 = make_uint4(0, 0, 0, 0);
  if (KB > 0) {
    load_stage(KB > 3 ? 3 : KB - 1, ra, rb);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(KB > 4 ? 4 : KB - 1, ra2, rb2);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  v8bf af[4], bfrag[JN];
  if (KB > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = read_a(0, i);
#pragma unroll
    for (int j = 0; j < JN; ++j) bfrag[j] = read_b(0, j);
  }

  // Ring of four bf16 stages: in the iteration for K-block kb (stage kb%4 is
  // already in registers), stage (kb+1)%4 is read for the next iteration
  // while this one computes, and stage (kb+3)%4 receives the K-block held in
  // registers.  A barrier after every second iteration orders them: a stage
  // written in iteration kb is read in iteration kb+2 at the earliest, and the
  // stage it overwrites was last read in iteration kb-2, both across a
  // barrier.  The loop runs four iterations per trip, so every stage offset
  // is a constant (measured 137 against 139 us at 4096^3 with three stages
  // and one barrier per K-block).

  // the scale products of the current K-block; those of the next are read
  // right after the last promotion, into the same registers, so the barrier
  // hides the LDS latency
  float s_cur[2][CBW];
  v4f_t sa4 = {0.0f, 0.0f, 0.0f, 0.0f}, s4 = {0.0f, 0.0f, 0.0f, 0.0f};
  float sbs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (KB > 0) {
    if constexpr (TG) read_tg_scales(0, sa4, sbs);
    else read_scales(0, s_cur);
  }
  // Two register sets alternate between iterations: the global loads of a
  // K-block (kb+5 in iteration kb) are issued two iterations before its
  // staging, so their latency hides behind two iterations of MFMAs.
  // `compute_tag` (std::true_type / std::false_type): false for a wave whose
  // row band holds no rows of the problem; it then only stages, refills the
  // scale windows and meets the barriers.
  auto iteration = [&](int kb, uint4& ra, uint4& rb, auto compute_tag, auto phase_tag) __attribute__((always_inline)) {
    constexpr bool COMPUTE = decltype(compute_tag)::value;
    constexpr int J = decltype(phase_tag)::value;        // kb % 4
    constexpr int sn = (J + 1) & 3, sf = (J + 3) & 3;    // stages of K-blocks kb+1 and kb+3
    // next window of scales: written now, first read SCW (SCWT) iterations later
    const bool tg_refill = TG && kb % SCWT == 0 && kb + SCWT < KB;
    if constexpr (TG) {
      if (tg_refill) load_tg_window(kb / SCWT + 1);
    } else {
      if (kb % SCW == 0 && kb + SCW < KB) load_scale_window(kb / SCW + 1);
    }

    // 32 sub-tile partials, j outer, so that each B fragment is dead after its
    // four uses and is refilled with the next K-block's.  The MFMAs run in
    // bursts of BU, each followed by the promotions of the burst before it, so
    // partials pass through a ring of 2 BU.  A SIMD runs two waves of the
    // tile, and a burst of MFMAs from one overlaps a burst of fmas from the
    // other: the probe's register-only loop of this mix at two waves per SIMD
    // took 26.6 cycles per MFMA and its four fmas interleaved, 24.6 in bursts
    // of two or three and 23.3 in bursts of six (bursts of four or more need
    // eight or more partials, which spill here; in this kernel bursts of
    // three beat bursts of two).  The staging of K-block kb+3 (decode + LDS stores) is cut
    // into four pieces spread over the MFMA sequence, so that no stretch of
    // the iteration is conversions alone.
    //
    // Wave priority falls in steps over the iteration (3 at its start, 0 from
    // the 30th of 32 MFMAs on; proportionally in a light tile).  At equal
    // priority the older wave of a SIMD issues first, runs ahead, and then
    // waits at the barrier while the other finishes alone.  Measured with
    // per-wave cycle counters at 4096^3: the leading waves waited 706 cycles
    // per K-block at the barrier, the others 106, in 2330-cycle K-blocks.
    // With the priority steps the wave that is behind in the iteration issues
    // first, the two stay close, and the kernel took 139 us against 145.
    constexpr int BU = 3;
    constexpr int PDEPTH = 2 * BU;
    constexpr int NG = (NQ + BU - 1) / BU;
    v4f pr[PDEPTH];
    if constexpr (!COMPUTE) {
      store_stage(sf, ra, rb);
      load_stage(kb + 5 < KB ? kb + 5 : KB - 1, ra, rb);
    }
    constexpr int QP2 = NQ * 10 / 32, QP1 = NQ * 20 / 32, QP0 = NQ * 30 / 32;  // priority steps
    constexpr int QS0 = NQ * 4 / 32, QS1 = NQ * 10 / 32, QS2 = NQ * 16 / 32, QS3 = NQ * 22 / 32;  // staging
    if constexpr (COMPUTE) __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int g = 0; g < (COMPUTE ? NG + 1 : 0); ++g) {
#pragma unroll
      for (int q = g * BU; q < (g + 1) * BU; ++q) {
        if (q >= NQ) break;
        if (q == QP2) __builtin_amdgcn_s_setprio(2);
        if (q == QP1) __builtin_amdgcn_s_setprio(1);
        if (q == QP0) __builtin_amdgcn_s_setprio(0);
        const int qi = q & 3, qj = q >> 2;
        pr[q % PDEPTH] = TG ? mfma_partial(bfrag[qj], af[qi]) : mfma_partial(af[qi], bfrag[qj]);
        if (qi == 3) bfrag[qj] = read_b(sn, qj);   // last use of this B fragment
        if (qj == JN - 1) af[qi] = read_a(sn, qi);  // last use of this A fragment
        // Unconditional (clamped) staging: a branch here would keep the old
        // and new register contents alive together.  Past the end the stage
        // written is never read.  Each register is reloaded (K-block kb+5) as
        // soon as both of its halves are staged, A before B as in the prologue.
        if (q == QS0) store_piece(sf, 0, ra, rb);
        if (q == QS1) {
          store_piece(sf, 1, ra, rb);
          load_a_only(kb + 5 < KB ? kb + 5 : KB - 1, ra);
        }
        if (q == QS2) store_piece(sf, 2, ra, rb);
        if (q == QS3) {
          store_piece(sf, 3, ra, rb);
          load_b_only(kb + 5 < KB ? kb + 5 : KB - 1, rb);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (g >= 1) {
#pragma unroll
        for (int u = (g - 1) * BU; u < g * BU; ++u) {
          if (u >= NQ) break;
          const int ui = u & 3, uj = u >> 2;
          if constexpr (TG) {
            if ((u & 7) == 0) s4 = sa4 * sbs[uj >> 1];  // this column block's four row scales
            promote(acc[ui][uj], pr[u % PDEPTH], s4[ui]);
          } else {
            promote(acc[ui][uj], pr[u % PDEPTH], s_cur[ui >> 1][uj >> 1]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (COMPUTE) {
      if constexpr (TG) read_tg_scales(kb + 1, sa4, sbs);
      else read_scales(kb + 1, s_cur);
    }
    // the window's direct loads (issued at the start of an even iteration)
    // have landed before the barrier that publishes them: only the operand
    // loads of that iteration and the next (four) were issued after them.
    if constexpr (J & 1) {
      if constexpr (TG) wait_vmcnt<4>();
      __syncthreads();
    }
  };
  // All four iterations of a trip are unconditional: a conditional one would
  // give the loop's back edge different orders of loads in flight, and the
  // compiler would then wait for all of them before staging.  KB is padded
  // to a multiple of four with empty K-blocks (kb >= KB) whose scale products
  // are zero: fma(P, 0, acc) returns acc for every nonzero acc, since P is
  // finite (a partial of finite codes).  A zero acc may change sign there;
  // the epilogue stores every exact zero as +0 (bf16_out), so the stored bits
  // equal those of a kernel that stops at the last K-block.
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  if (p.row0 + wm * 64 < p.row_end) {   // this wave's row band holds rows of the problem
    for (int kb = 0; kb < KB; kb += 4) {
      iteration(kb, ra, rb, std::true_type{}, P0{});
      iteration(kb + 1, ra2, rb2, std::true_type{}, P1{});
      iteration(kb + 2, ra, rb, std::true_type{}, P2{});
      iteration(kb + 3, ra2, rb2, std::true_type{}, P3{});
    }
  } else {
    for (int kb = 0; kb < KB; kb += 4) {
      iteration(kb, ra, rb, std::false_type{}, P0{});
      iteration(kb + 1, ra2, rb2, std::false_type{}, P1{});
      iteration(kb + 2, ra, rb, std::false_type{}, P2{});
      iteration(kb + 3, ra2, rb2, std::false_type{}, P3{});
    }
  }

  // ---- epilogue: bf16, through LDS (per-wave 32 x WN_T region, two passes) for
  // 16-byte coalesced global stores
  constexpr int EP_ROW = WN_T * 2;        // bytes per row of the region
  constexpr int EP_LPR = WN_T / 8;        // lanes per row in the store pass
  unsigned char* ep = smem + w * (32 * EP_ROW);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = pass * 2 + ii;
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        if constexpr (TG) {
          // lane holds row ii*16 + (lane&15), columns j*16 + 4*(lane>>4) + 0..3
          const int lr = ii * 16 + (lane & 15);
          const int lc = j * 16 + 4 * (lane >> 4);
          const uint32_t lo = bf16_out(acc[i][j][0]) | (bf16_out(acc[i][j][1]) << 16);
          const uint32_t hi = bf16_out(acc[i][j][2]) | (bf16_out(acc[i][j][3]) << 16);
          *reinterpret_cast<uint2*>(ep + lr * EP_ROW + lc * 2) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int lr = ii * 16 + 4 * (lane >> 4) + r;
            const int lc = j * 16 + (lane & 15);
            *reinterpret_cast<uint16_t*>(ep + lr * EP_ROW + lc * 2) = (uint16_t)bf16_out(acc[i][j][r]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 32 * EP_LPR / 64; ++it) {
      const int lr = it * (64 / EP_LPR) + lane / EP_LPR;
      const int lc = (lane % EP_LPR) * 8;
      uint4 v = *reinterpret_cast<const uint4*>(ep + lr * EP_ROW + lc * 2);
      const int64_t grow = p.row0 + wm * 64 + pass * 32 + lr;
      const int64_t gcol = p.col0 + wn * WN_T + lc;
      if (grow < p.row_end && gcol < N) *reinterpret_cast<uint4*>(p.c + grow * N + gcol) = v;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <bool BT, bool TG>
__global__ void __launch_bounds__(TTHREADS) gemm_tile_kernel(const uint8_t* __restrict__ a,
                                                             const float* __restrict__ sa,
                                                             const uint8_t* __restrict__ b,
                                                             const float* __restrict__ sb, uint16_t* __restrict__ c,
                                                             int64_t M, int64_t N, int64_t K, int64_t tiles_m,
                                                             int64_t tiles_n, int remap) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int64_t n_tiles = tiles_m * tiles_n;
  int64_t tm, tn;
  if (remap) {
    tile_coords(blockIdx.x, n_tiles, tiles_n, tm, tn);
  } else {
    tm = blockIdx.x / tiles_n;
    tn = blockIdx.x % tiles_n;
  }
  TileArgs p;
  p.a = a;
  p.sa = sa;
  p.b = b;
  p.sb = sb;
  p.c = c;
  p.N = N;
  p.K = K;
  p.row0 = tm * TBM;
  p.row_end = M;
  p.col0 = tn * TBN;
  p.sa_rows = (M + 31) >> 5;
  if constexpr (!TG) {
    // a last M-tile of at most 128 rows runs as a light tile
    if (M - p.row0 <= 128) tile_body<BT, TG, true>(p, smem);
    else tile_body<BT, TG>(p, smem);
  } else {
    tile_body<BT, TG>(p, smem);
  }
}

// Grouped GEMM (DeepGEMM write-up, sections 4.1-4.3): group g owns rows
// [off_g, off_{g+1}) of A and C and multiplies them by B_g.  The offsets stay
// in device memory and are read by the kernel, so a launch's arguments never
// depend on the group sizes.
//
// Load balance (section 4.2): every group's rows are cut into 256-row tiles;
// a group's last tile may be partial.  A tile with more than 128 rows keeps
// every SIMD busy for the whole tile ("heavy"); one with at most 128 rows
// leaves half of the waves idle and takes about half the time ("light";
// measured 211 against 394 us per tile at K = 7168).  Workgroup i takes tile i
// of a list that holds every heavy tile first and every light one after them
// (each group-major, column tiles innermost); the hardware hands out
// workgroups in index order as CUs free up, so the cheap tiles fill the last
// wave.  Measured on 16 groups of ~585 rows: 0.68 ms against 0.77 ms with
// each group's tiles kept together.  The grid is an upper bound on the tile
// count; workgroups past the list leave at once.  Every tile is computed by
// tile_body exactly as in a plain GEMM.

// Wave-wide inclusive scans over the 64 lanes (the tile lookup only).
__device__ __forceinline__ long long wave_incl_sum(long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}
__device__ __forceinline__ long long wave_incl_max(long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long o = __shfl_up(v, d, 64);
    if (lane >= d && o > v) v = o;
  }
  return v;
}

// Walks the groups 64 at a time (one lane per group).  Offsets are clamped to
// [0, M_total] and ranges that overlap an earlier group's are clipped, so the
// rows of group g are [s0_g, s1_g) with s0_g = max(c_0..c_g) and
// s1_g = max(s0_g, c_{g+1}), c = the clamped offsets.  With want < 0 it only
// counts: returns the number of heavy (cls 0) or light (cls 1) M-tiles.  With
// want >= 0 it finds the want-th M-tile of class cls and returns its group
// and rows (-1 if there is none).  Every lane returns the same values.
__device__ long long grouped_walk(const int32_t* __restrict__ offsets, int G, int64_t M_total, int cls,
                                  long long want, int& g_out, int64_t& start, int64_t& end) {
  const int lane = threadIdx.x & 63;
  long long run_max = 0, base = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    const bool valid = g < G;
    long long c0 = valid ? offsets[g] : 0, c1 = valid ? offsets[g + 1] : 0;
    c0 = c0 < 0 ? 0 : (c0 > M_total ? M_total : c0);
    c1 = c1 < 0 ? 0 : (c1 > M_total ? M_total : c1);
    long long s0 = wave_incl_max(c0);
    s0 = s0 > run_max ? s0 : run_max;
    const long long s1 = c1 > s0 ? c1 : s0;
    const long long rows = valid ? s1 - s0 : 0;
    const long long full = rows >> 8, rem = rows & (TBM - 1);
    const long long cnt = cls == 0 ? full + (rem > TBM / 2 ? 1 : 0) : (rem > 0 && rem <= TBM / 2 ? 1 : 0);
    const long long incl = wave_incl_sum(cnt);
    const long long excl = incl - cnt;
    if (want >= 0) {
      const bool hit = cnt > 0 && want >= base + excl && want < base + incl;
      const unsigned long long mask = __ballot(hit);
      if (mask) {
        const int src = __ffsll((long long)mask) - 1;
        const long long my_start = cls == 0 ? s0 + (want - base - excl) * TBM : s0 + full * TBM;
        start = __shfl(my_start, src, 64);
        end = __shfl(s1, src, 64);
        g_out = g0 + src;
        return 0;
      }
    }
    base += __shfl(incl, 63, 64);
    run_max = __shfl(s0, 63, 64);
  }
  return want >= 0 ? -1 : base;
}

template <bool BT>
__global__ void __launch_bounds__(TTHREADS) gemm_grouped_kernel(const uint8_t* __restrict__ a,
                                                                const float* __restrict__ sa,
                                                                const uint8_t* __restrict__ b,
                                                                const float* __restrict__ sb,
                                                                const int32_t* __restrict__ offsets, int G,
                                                                uint16_t* __restrict__ c, int64_t M_total, int64_t N,
                                                                int64_t K, int64_t tiles_n) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int g = 0;
  int64_t start = 0, end = 0;
  const long long heavy = grouped_walk(offsets, G, M_total, 0, -1, g, start, end);
  const long long light = grouped_walk(offsets, G, M_total, 1, -1, g, start, end);
  const long long n_heavy = heavy * tiles_n, total = (heavy + light) * tiles_n;
  const int64_t KB = K >> 5, NB = N >> 5;
  {
    const long long i = blockIdx.x;
    if (i >= total) return;
    const int cls = i < n_heavy ? 0 : 1;
    const long long r = cls == 0 ? i : i - n_heavy;
    const long long mt = r / tiles_n, tn = r % tiles_n;
    if (grouped_walk(offsets, G, M_total, cls, mt, g, start, end) < 0) return;
    TileArgs p;
    p.a = a;
    p.sa = sa;
    p.b = b + (int64_t)g * K * N;
    p.sb = sb + (int64_t)g * KB * NB;
    p.c = c;
    p.N = N;
    p.K = K;
    p.row0 = start;
    p.row_end = end;
    p.col0 = tn * TBN;
    p.sa_rows = M_total >> 5;
    if (cls == 0) tile_body<BT, false>(p, smem);
    else tile_body<BT, false, true>(p, smem);
  }
}

// ------------------------------------------------------------------------------------
// small-M kernel
// ------------------------------------------------------------------------------------
constexpr int SWAVES = 8;        // waves per workgroup; also K-blocks per round
constexpr int STHREADS = SWAVES * 64;
constexpr int SMALL_LDS_BUDGET = 160 * 1024;

// Small-M kernel: a workgroup owns W = 32*NCB columns of C for all M <= 64
// rows and all of K.  K-blocks are streamed in rounds of eight: in round r,
// wave q loads K-block 8r+q (B tile 32 x W bytes, the A rows, the scales) into
// its own slot of an LDS ring D rounds deep.  After one barrier every wave
// reads all eight slots and runs the promotion chain of the 16x16 output
// sub-tiles it owns, K-block by K-block in ascending order, so no partial
// result ever crosses waves.
//
// B tile layout in a slot: row k (32 rows of W bytes), 16-byte piece p holds
// global piece p ^ f(k), where f(k) = (k / (256/W)) mod (2*NCB): the sixteen
// rows that one 32-lane phase of a transposed read touches land in sixteen
// different 16-byte bank groups.
template <int MT, int NCB, bool TG = false>
struct SmallMCfg {
  static constexpr int W = 32 * NCB;                   // columns (= bytes of a B row) per workgroup
  static constexpr int ACH = (MT + 1) / 2;             // 1 KB chunks of A rows (32 rows each)
  static constexpr int B_BYTES = 32 * W;
  static constexpr int SC_OFF = B_BYTES + ACH * 1024;  // scale record(s) after B and A
  // block scales: one 256-byte record (sa of 2 row-blocks, sb); token-group
  // scales: sa of every row (256 bytes), then sb (256 bytes)
  // token-group scales with at most 32 rows: one packed record (lanes 0-31 sa
  // of rows 0-31, lanes 32.. sb of the column blocks)
  static constexpr bool TG_PACKED = TG && MT <= 2;
  static constexpr int SLOT = SC_OFF + (TG && !TG_PACKED ? 512 : 256);
  // 32x32 scales: wave 0 loads the whole round's scale record (sa of up to
  // two row-blocks and sb of the slice's column blocks for eight K-blocks)
  // with one direct load; token-group records stay one per wave and K-block
  static constexpr bool ROUND_SC = !TG;
  static constexpr int OPS = NCB + ACH + (TG && !TG_PACKED ? 2 : 1);  // direct loads per K-block (wave 0)
  static constexpr int OPS_OTHER = ROUND_SC ? NCB + ACH : OPS;        // the other waves
  static constexpr int CS = 2 * NCB;                   // 16-column sub-tiles per workgroup
  static constexpr int RG = SWAVES / CS;               // row-tile groups
  static constexpr int TPW = (MT + RG - 1) / RG;       // row tiles per wave (at most)
  // Shared bf16 A: where a wave owns two or more row tiles of one A chunk
  // (17-32 rows, 128-column slices), every wave decodes only the A chunk it
  // loaded into a bf16 area shared by the workgroup, [2 rounds][8 K-blocks]
  // [32 rows][64 B], instead of decoding every K-block's A fragments itself
  // (measured 59.5 against 69.5 us at M = 32, N = 28672; with one row tile
  // per wave the extra LDS round trip cost 1-5%).  Only where the ring still
  // gets three rounds.
  static constexpr int ABUF_FULL = 2 * SWAVES * 32 * 64;
  static constexpr bool A_SHARED =
      ACH == 1 && TPW >= 2 && (SMALL_LDS_BUDGET - ABUF_FULL) / (SWAVES * SLOT) >= 3;
  static constexpr int ABUF_BYTES = A_SHARED ? ABUF_FULL : 0;
  static constexpr int D_FIT = (SMALL_LDS_BUDGET - ABUF_BYTES) / (SWAVES * SLOT);
  static constexpr int D = D_FIT > 6 ? 6 : D_FIT;      // ring depth in rounds
  static constexpr int ABUF_OFF = SWAVES * D * SLOT;
  static constexpr int LDS = ABUF_OFF + ABUF_BYTES;
  static_assert(D >= 3, "ring too shallow");
  static_assert(LDS <= SMALL_LDS_BUDGET, "LDS budget");
  static_assert((D - 2) * OPS < 64, "vmcnt range");
};

template <int NCB>
__device__ __forceinline__ int small_b_swz(int k) {
  return (k / (8 / NCB)) & (2 * NCB - 1);
}

template <int MT, int NCB, bool TG>
__global__ void __launch_bounds__(STHREADS) gemm_smallm_kernel(const uint8_t* __restrict__ a,
                                                               const float* __restrict__ sa,
                                                               const uint8_t* __restrict__ b,
                                                               const float* __restrict__ sb,
                                                               uint16_t* __restrict__ c, int64_t M, int64_t N,
                                                               int64_t K) {
  using Cfg = SmallMCfg<MT, NCB, TG>;
  constexpr int D = Cfg::D, W = Cfg::W;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int w = wave_id_uniform();
  const int KB = (int)(K >> 5), NB = (int)(N >> 5);
  // Workgroups on one XCD (blockIdx mod 8) take adjacent column slices, so the
  // 128-byte lines of B that narrow slices share are fetched into that XCD's L2 once.
  const int64_t n_slices = N / W;
  const int64_t id = blockIdx.x;
  const int64_t slice = (n_slices & 7) ? id : (id & 7) * (n_slices >> 3) + (id >> 3);
  const int64_t n0 = slice * W;
  const int cb0 = (int)(n0 >> 5);

  // ---- this wave's direct loads for one K-block ----
  // B: instruction i covers rows i*(32/NCB) ... ; lane l -> row k, LDS piece p.
  constexpr int LPR = W / 16;  // lanes per B row
  const uint8_t* b_src[NCB];
#pragma unroll
  for (int i = 0; i < NCB; ++i) {
    const int k = i * (64 / LPR) + lane / LPR, p = lane % LPR;
    b_src[i] = b + (int64_t)k * N + n0 + 16 * (p ^ small_b_swz<NCB>(k));
  }
  // A: chunk ch covers rows 32ch..32ch+31; lane l loads row 32ch + (l>>1),
  // 16-byte half l&1.  Rows past M read row M-1: their results are never stored.
  const uint8_t* a_src[Cfg::ACH];
#pragma unroll
  for (int ch = 0; ch < Cfg::ACH; ++ch) {
    int64_t row = ch * 32 + (lane >> 1);
    row = row < M ? row : M - 1;
    a_src[ch] = a + row * K + (lane & 1) * 16;
  }
  const int nrb = (int)((M + 31) >> 5);
  // round record (wave 0): lane l < 16 = sa of row-block min(l >> 3, nrb-1) at
  // K-block 8r + (l & 7); lane 16 + 8j' .. = sb of column block cb0 + c at
  // K-block 8r + q for l - 16 = q * NCB + c (lanes past 16 + 8*NCB repeat the
  // last entry); every address is clamped to the last K-block
  const int rs_l = lane < 16 ? lane : (lane - 16 < 8 * NCB ? lane - 16 : 8 * NCB - 1);
  const int rs_q = lane < 16 ? (rs_l & 7) : rs_l / NCB;
  const float* const rs_src = lane < 16 ? sa + (int64_t)((lane >> 3) < nrb ? (lane >> 3) : nrb - 1) * KB
                                        : sb + cb0 + rs_l % NCB;
  const int64_t rs_stride = lane < 16 ? 1 : NB;
  // token-group scales: record 1, lane l = sa of row min(l, M-1); record 2,
  // lane l = sb of column block cb0 + min(l, NCB-1)
  const float* const tg_sa_src = sa + (int64_t)(lane < M ? lane : M - 1) * KB;
  const float* const tg_sb_src = sb + cb0 + (lane < NCB ? lane : NCB - 1);
  // packed record (M <= 32): lane l < 32 = sa of row min(l, M-1), lane 32 + j =
  // sb of column block cb0 + min(j, NCB-1); sa steps 1, sb steps NB per K-block
  const float* const tg_pk_src = lane < 32 ? sa + (int64_t)(lane < M ? lane : M - 1) * KB
                                           : sb + cb0 + (lane - 32 < NCB ? lane - 32 : NCB - 1);
  const int64_t tg_pk_stride = lane < 32 ? 1 : NB;
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  const uint32_t ring_w = (uint32_t)(uintptr_t)((lds_u8*)(smem + w * D * Cfg::SLOT));

  auto issue = [&](int r) __attribute__((always_inline)) {
    const int kb = r * SWAVES + w;
    const int kc = kb < KB ? kb : KB - 1;  // past the end: reload the last block (an L2 hit)
    const uint32_t sl = ring_w + (r % D) * Cfg::SLOT;
#pragma unroll
    for (int i = 0; i < NCB; ++i) dma16(b_src[i] + (int64_t)kc * 32 * N, sl + i * 1024);
#pragma unroll
    for (int ch = 0; ch < Cfg::ACH; ++ch) dma16(a_src[ch] + (int64_t)kc * 32, sl + Cfg::B_BYTES + ch * 1024);
    if constexpr (Cfg::TG_PACKED) {
      dma4(tg_pk_src + (int64_t)kc * tg_pk_stride, sl + Cfg::SC_OFF);
    } else if constexpr (TG) {
      dma4(tg_sa_src + kc, sl + Cfg::SC_OFF);
      dma4(tg_sb_src + (int64_t)kc * NB, sl + Cfg::SC_OFF + 256);
    } else {
      if (w == 0) {
        int kr = r * SWAVES + rs_q;
        kr = kr < KB ? kr : KB - 1;
        dma4(rs_src + (int64_t)kr * rs_stride, sl + Cfg::SC_OFF);
      }
    }
  };

  // ---- ownership: 16-column sub-tile cs, row tiles rg, rg + RG, ... ----
  const int cs = w % Cfg::CS;
  const int rg = Cfg::RG == 1 ? 0 : w / Cfg::CS;
  const int own_cb = cs >> 1;  // column block (within the slice) of the sub-tile
  const bool owns = rg < MT;   // wave-uniform: waves past the last row tile only load
  // row tile of slot t; a wave's slots past the last row tile repeat it (never stored)
  auto tile_of = [&](int t) __attribute__((always_inline)) {
    const int i = rg + t * Cfg::RG;
    return i < MT ? i : MT - 1;
  };
  v4f acc[Cfg::TPW];
#pragma unroll
  for (int t = 0; t < Cfg::TPW; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // transposed-read address of this lane's B fragment inside a slot
  const int L = lane & 15;
  const int bk = 8 * (lane >> 4) + (L >> 1);
  const int b_frag_off = bk * W + 16 * (cs ^ small_b_swz<NCB>(bk)) + 8 * (L & 1);
  const int a_frag_off = Cfg::B_BYTES + (lane & 15) * 32 + (lane >> 4) * 8;

  // Shared bf16 A (M <= 32): row r's 16-byte chunk c (K elements 8c..8c+7) of
  // K-block q sits at chunk position c ^ ((r >> 1) & 3) of the row's 64 bytes.
  // Wave w decodes its own slot's chunk (lane l: row l >> 1, bytes 16*(l & 1))
  // after its loads have landed and before the round's barrier.
  auto abuf_off = [](int row, int chunk) __attribute__((always_inline)) {
    return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4);
  };
  auto decode_own_a = [&](int r) __attribute__((always_inline)) {
    const unsigned char* src =
        smem + (w * D + r % D) * Cfg::SLOT + Cfg::B_BYTES + (lane >> 1) * 32 + (lane & 1) * 16;
    uint4 lo, hi;
    e4m3x16_to_bf16x16(*reinterpret_cast<const uint4*>(src), lo, hi);
    unsigned char* dst = smem + Cfg::ABUF_OFF + ((r & 1) * SWAVES + w) * 2048;
    *reinterpret_cast<uint4*>(dst + abuf_off(lane >> 1, 2 * (lane & 1))) = lo;
    *reinterpret_cast<uint4*>(dst + abuf_off(lane >> 1, 2 * (lane & 1) + 1)) = hi;
  };

  // One round: all LDS reads first, then per K-block q (ascending) the MFMA
  // partials of the owned tiles and their promotion.  FULL: all eight K-blocks
  // exist (every round but possibly the last).
  auto compute = [&](int r, int nkb, auto FULL_) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(FULL_)::value;
    const int slot = r % D;
    v2i braw[SWAVES];
    v2i araw[SWAVES][Cfg::TPW];
    v8bf abf[SWAVES][Cfg::TPW];
    float sbv[SWAVES], sav[SWAVES][2], sat[SWAVES][Cfg::TPW];
#pragma unroll
    for (int q = 0; q < SWAVES; ++q) {
      const unsigned char* sl = smem + (q * D + slot) * Cfg::SLOT;
      braw[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(sl + b_frag_off));
#pragma unroll
      for (int t = 0; t < Cfg::TPW; ++t) {
        if constexpr (Cfg::A_SHARED) {
          const unsigned char* ab = smem + Cfg::ABUF_OFF + ((r & 1) * SWAVES + q) * 2048;
          abf[q][t] = *reinterpret_cast<const v8bf*>(ab + abuf_off(16 * tile_of(t) + (lane & 15), lane >> 4));
        } else {
          araw[q][t] = *reinterpret_cast<const v2i*>(sl + a_frag_off + tile_of(t) * 16 * 32);
        }
      }
      const float* scr = reinterpret_cast<const float*>(sl + Cfg::SC_OFF);
      if constexpr (TG) {
        // this lane's row scale in each owned row tile (rows 16*i + (lane&15))
#pragma unroll
        for (int t = 0; t < Cfg::TPW; ++t) sat[q][t] = scr[16 * tile_of(t) + (lane & 15)];
        sbv[q] = scr[(Cfg::TG_PACKED ? 32 : 64) + own_cb];
      } else {
        // the round record in wave 0's slot
        const float* rec = reinterpret_cast<const float*>(smem + slot * Cfg::SLOT + Cfg::SC_OFF);
        sav[q][0] = rec[q];
        sav[q][1] = rec[8 + q];
        sbv[q] = rec[16 + q * NCB + own_cb];
      }
    }
    // K-block q's partials are promoted after K-block q+1's MFMAs are issued,
    // so no fma waits on the MFMA right before it; each acc[t] still takes the
    // K-blocks in ascending order (the same bits).  Measured at K = 8192:
    // N = 28672, M = 32 / 48 / 64 62.1 / 82.5 / 104.9 -> 60.1 / 77.9 / 97.3 us,
    // M <= 16 unchanged.  (The K-major kernel measured slower this way at
    // M = 64, N = 28672: 93.8 against 86.7 us.)
    v4f pp[2][Cfg::TPW];
    float psc[2][Cfg::TPW];
#pragma unroll
    for (int q = 0; q <= SWAVES; ++q) {
      if (q < SWAVES) {
        const v8bf bfrag = e4m3x8_to_bf16x8(braw[q]);
#pragma unroll
        for (int t = 0; t < Cfg::TPW; ++t) {
          const v8bf afrag = Cfg::A_SHARED ? abf[q][t] : e4m3x8_to_bf16x8(araw[q][t]);
          pp[q & 1][t] = TG ? mfma_partial(bfrag, afrag) : mfma_partial(afrag, bfrag);
          psc[q & 1][t] = (TG ? sat[q][t] : sav[q][tile_of(t) >> 1]) * sbv[q];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (q > 0) {
#pragma unroll
        for (int t = 0; t < Cfg::TPW; ++t)
          if (FULL || q - 1 < nkb) promote(acc[t], pp[(q - 1) & 1][t], psc[(q - 1) & 1][t]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int rounds = (KB + SWAVES - 1) / SWAVES;
  const int full_rounds = KB / SWAVES;
  // K = 0: nothing is loaded (the caller may pass null pointers); zeros are stored.
  if (KB > 0) {
#pragma unroll
    for (int d = 0; d < D - 1; ++d) issue(d);
  }

  for (int r = 0; r < rounds; ++r) {
    // this wave's round-r loads have landed
    if (w == 0) wait_vmcnt<(D - 2) * Cfg::OPS>();
    else wait_vmcnt<(D - 2) * Cfg::OPS_OTHER>();
    // the shared A area of round r - 2 is free: every wave finished that
    // round's compute before the previous barrier
    if constexpr (Cfg::A_SHARED) decode_own_a(r);
    lds_barrier();                     // ... and everyone else's; round r-1's slots are free
    issue(r + D - 1);                  // refill the slot that round r-1 used
    if (owns) {
      if (r < full_rounds) compute(r, SWAVES, std::true_type{});
      else compute(r, KB - r * SWAVES, std::false_type{});
    }
  }
  wait_vmcnt<0>();  // drain the extra loads before the workgroup ends

#pragma unroll
  for (int t = 0; t < Cfg::TPW; ++t) {
    const int i = rg + t * Cfg::RG;
    if (owns && i < MT) {
      if constexpr (TG) {
        // lane holds row 16*i + (lane&15), columns cs*16 + 4*(lane>>4) + 0..3
        const int64_t row = i * 16 + (lane & 15);
        const int64_t col4 = n0 + cs * 16 + 4 * (lane >> 4);
        if (row < M) {
          const uint32_t lo = bf16_out(acc[t][0]) | (bf16_out(acc[t][1]) << 16);
          const uint32_t hi = bf16_out(acc[t][2]) | (bf16_out(acc[t][3]) << 16);
          *reinterpret_cast<uint2*>(c + row * N + col4) = make_uint2(lo, hi);
        }
      } else {
        const int col = (int)n0 + cs * 16 + (lane & 15);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int64_t row = i * 16 + 4 * (lane >> 4) + rr;
          if (row < M) c[row * N + col] = (uint16_t)bf16_out(acc[t][rr]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// small-M kernel, K-major weight (B^T [N, K], scales [NB, KB])
// ------------------------------------------------------------------------------------
// The workgroup's W = 32*NCB columns of C are W contiguous rows of B^T, so each
// round streams W rows x 256 bytes (eight K-blocks) and every row is read as
// whole 256-byte runs.  Round buffer layout (one per ring slot): the W weight
// rows, then the 32*ACH A rows, each 256 bytes with 16-byte piece p of row r
// holding global piece p ^ (r & 15) (the fragment reads of sixteen rows at one
// K offset then hit sixteen bank groups), then eight 256-byte scale records
// (record q: sa of row-blocks 0 and 1, sb of the NCB column blocks, for K-block
// 8r+q).  Every wave issues NCB 1 KB weight loads, ACH 1 KB A loads and one
// scale record per round.
template <int MT, int NCB, bool TG = false>
struct SmallMNtCfg {
  static constexpr int W = 32 * NCB;
  static constexpr int ACH = (MT + 1) / 2;
  static constexpr int A_OFF = W * 256;
  static constexpr int SC_OFF = A_OFF + 32 * ACH * 256;
  // token-group scales with at most 32 rows: one packed record, as in the
  // [K, N] kernel
  static constexpr bool TG_PACKED = TG && MT <= 2;
  static constexpr int REC = TG && !TG_PACKED ? 512 : 256;  // scale record per K-block (token groups: sa rows, then sb)
  static constexpr int SLOT = SC_OFF + SWAVES * REC;
  static constexpr int OPS = NCB + ACH + (TG && !TG_PACKED ? 2 : 1);
  // 32x32 scales: wave 0 loads the whole round's scale record with one direct
  // load (as in the [K, N] kernel); SCL = scale loads per round of the other waves
  static constexpr bool ROUND_SC = !TG;
  static constexpr int SCL = ROUND_SC ? 0 : (TG && !TG_PACKED ? 2 : 1);
  static constexpr int CS = 2 * NCB;
  static constexpr int RG = SWAVES / CS;
  static constexpr int TPW = (MT + RG - 1) / RG;
  // Shared bf16 A, as in the [K, N] kernel: where a wave owns two or more row
  // tiles of one A chunk, each wave decodes the four A rows it loaded into a
  // double-buffered bf16 area [2 rounds][32 rows][8 K-blocks x 64 B].
  static constexpr int ABUF_FULL = 2 * 32 * SWAVES * 64;
  static constexpr bool A_SHARED = ACH == 1 && TPW >= 2 && (SMALL_LDS_BUDGET - ABUF_FULL) / SLOT >= 3;
  static constexpr int ABUF_BYTES = A_SHARED ? ABUF_FULL : 0;
  static constexpr int D_FIT = (SMALL_LDS_BUDGET - ABUF_BYTES) / SLOT;
  static constexpr int D = D_FIT > 6 ? 6 : D_FIT;
  static constexpr int ABUF_OFF = D * SLOT;
  static constexpr int LDS = ABUF_OFF + ABUF_BYTES;
  static_assert(D >= 3, "ring too shallow");
  static_assert(LDS <= SMALL_LDS_BUDGET, "LDS budget");
  static_assert((D - 2) * OPS < 64, "vmcnt range");
};

template <int MT, int NCB, bool TG>
__global__ void __launch_bounds__(STHREADS) gemm_smallm_nt_kernel(const uint8_t* __restrict__ a,
                                                                  const float* __restrict__ sa,
                                                                  const uint8_t* __restrict__ bt,
                                                                  const float* __restrict__ sbt,
                                                                  uint16_t* __restrict__ c, int64_t M, int64_t N,
                                                                  int64_t K) {
  using Cfg = SmallMNtCfg<MT, NCB, TG>;
  constexpr int D = Cfg::D, W = Cfg::W;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int w = wave_id_uniform();
  const int KB = (int)(K >> 5);
  const int64_t n_slices = N / W;
  const int64_t slice = blockIdx.x;
  const int64_t n0 = slice * W;
  const int cb0 = (int)(n0 >> 5);

  // ---- this wave's direct loads for round r
  // weight piece i: rows 4*(w*NCB + i) .. +3; lane l -> row 4*(w*NCB+i) + l/16, LDS piece l%16
  const int lp = lane & 15;
  const uint8_t* b_row[NCB];
  int b_g[NCB];
#pragma unroll
  for (int i = 0; i < NCB; ++i) {
    const int r = 4 * (w * NCB + i) + (lane >> 4);
    b_row[i] = bt + (n0 + r) * K;
    b_g[i] = lp ^ (r & 15);
  }
  // A piece ch: rows 4*(w + 8*ch) .. +3 (rows past M read row M-1).  A piece
  // whose four rows all lie past M is not loaded at all: an MFMA output row
  // depends only on its own A row, and rows past M are never stored, so
  // whatever their LDS bytes hold cannot reach C.  a_live (wave-uniform) counts
  // this wave's loaded pieces; they are the first a_live values of ch.
  const uint8_t* a_row[Cfg::ACH];
  int a_g[Cfg::ACH];
  int a_live = 0;
#pragma unroll
  for (int ch = 0; ch < Cfg::ACH; ++ch) {
    const int r = 4 * (w + 8 * ch) + (lane >> 4);
    const int64_t rr = r < M ? r : M - 1;
    a_row[ch] = a + rr * K;
    a_g[ch] = lp ^ (r & 15);
    a_live += 4 * (w + 8 * ch) < M ? 1 : 0;
  }
  const int nrb = (int)((M + 31) >> 5);
  // round record (wave 0): lane l < 16 = sa of row-block min(l >> 3, nrb-1) at
  // K-block 8r + (l & 7); lane 16 + q*NCB + c = sbt of column block cb0 + c at
  // K-block 8r + q (lanes past 16 + 8*NCB repeat the last entry); both step 1
  // per K-block, and every K-block index is clamped to the last one
  const int rs_l = lane < 16 ? lane : (lane - 16 < 8 * NCB ? lane - 16 : 8 * NCB - 1);
  const int rs_q = lane < 16 ? (rs_l & 7) : rs_l / NCB;
  const float* const rs_src = lane < 16 ? sa + (int64_t)((lane >> 3) < nrb ? (lane >> 3) : nrb - 1) * KB
                                        : sbt + (int64_t)(cb0 + rs_l % NCB) * KB;
  // token-group scales: record 1, lane l = sa of row min(l, M-1); record 2,
  // lane l = sbt of column block cb0 + min(l, NCB-1)
  const float* const tg_sa_src = sa + (int64_t)(lane < M ? lane : M - 1) * KB;
  const float* const tg_sb_src = sbt + (int64_t)(cb0 + (lane < NCB ? lane : NCB - 1)) * KB;
  // packed record (M <= 32): lane l < 32 = sa of row min(l, M-1), lane 32 + j =
  // sbt of column block cb0 + min(j, NCB-1); both step 1 per K-block
  const float* const tg_pk_src =
      lane < 32 ? tg_sa_src : sbt + (int64_t)(cb0 + (lane - 32 < NCB ? lane - 32 : NCB - 1)) * KB;
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  const uint32_t ring = (uint32_t)(uintptr_t)((lds_u8*)smem);

  // byte offset in a row of global piece g of round r; pieces of K-blocks past
  // the end re-read the last K-block (their results are never used)
  auto koff = [&](int r, int g) __attribute__((always_inline)) -> int64_t {
    int kb = r * SWAVES + (g >> 1);
    kb = kb < KB ? kb : KB - 1;
    return (int64_t)kb * 32 + (g & 1) * 16;
  };
  auto issue = [&](int r) __attribute__((always_inline)) {
    const uint32_t sl = ring + (r % D) * Cfg::SLOT;
#pragma unroll
    for (int i = 0; i < NCB; ++i) dma16(b_row[i] + koff(r, b_g[i]), sl + (w * NCB + i) * 1024);
#pragma unroll
    for (int ch = 0; ch < Cfg::ACH; ++ch)
      if (ch < a_live) dma16(a_row[ch] + koff(r, a_g[ch]), sl + Cfg::A_OFF + (w + 8 * ch) * 1024);
    int kc = r * SWAVES + w;
    kc = kc < KB ? kc : KB - 1;
    if constexpr (Cfg::TG_PACKED) {
      dma4(tg_pk_src + kc, sl + Cfg::SC_OFF + w * Cfg::REC);
    } else if constexpr (TG) {
      dma4(tg_sa_src + kc, sl + Cfg::SC_OFF + w * Cfg::REC);
      dma4(tg_sb_src + kc, sl + Cfg::SC_OFF + w * Cfg::REC + 256);
    } else {
      if (w == 0) {
        int kr = r * SWAVES + rs_q;
        kr = kr < KB ? kr : KB - 1;
        dma4(rs_src + kr, sl + Cfg::SC_OFF);
      }
    }
  };

  // ---- ownership (as in the [K, N] kernel): 16-column sub-tile cs, row tiles rg, rg + RG, ...
  const int cs = w % Cfg::CS;
  const int rg = Cfg::RG == 1 ? 0 : w / Cfg::CS;
  const int own_cb = cs >> 1;
  const bool owns = rg < MT;
  auto tile_of = [&](int t) __attribute__((always_inline)) {
    const int i = rg + t * Cfg::RG;
    return i < MT ? i : MT - 1;
  };
  v4f acc[Cfg::TPW];
#pragma unroll
  for (int t = 0; t < Cfg::TPW; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // fragment of K-block q: lane l reads row (16*x + (l&15)), bytes 32q + 8*(l>>4):
  // piece 2q + (l>>5), half (l>>4)&1; row & 15 = l & 15 for every such row
  const int fr_half = ((lane >> 4) & 1) * 8, fr_hi = lane >> 5;
  auto frag_off = [&](int row, int q) __attribute__((always_inline)) {
    return row * 256 + 16 * ((2 * q + fr_hi) ^ (lane & 15)) + fr_half;
  };

  // Shared bf16 A: row R's 16-byte bf16 piece p (K-block p >> 2, K elements
  // 8*(p & 3) ..) sits at position p ^ (R & 15) of the row's 512 bytes.  Wave w
  // decodes its own rows 4w .. 4w + 3 (lane l: row 4w + (l >> 4), the raw piece
  // at position l & 15, i.e. global piece (l & 15) ^ (R & 15)) after its loads
  // have landed and before the round's barrier; rows past M are not loaded
  // and not decoded (they only reach outputs that are never stored).
  auto decode_own_a = [&](int r) __attribute__((always_inline)) {
    if (a_live == 0) return;
    const int R = 4 * w + (lane >> 4);
    const int g = (lane & 15) ^ (R & 15);
    const unsigned char* src = smem + (r % D) * Cfg::SLOT + Cfg::A_OFF + w * 1024 + lane * 16;
    uint4 lo, hi;
    e4m3x16_to_bf16x16(*reinterpret_cast<const uint4*>(src), lo, hi);
    unsigned char* dst = smem + Cfg::ABUF_OFF + (r & 1) * (32 * 512) + R * 512;
    const int p0 = 4 * (g >> 1) + 2 * (g & 1);
    *reinterpret_cast<uint4*>(dst + ((p0 ^ (R & 15)) << 4)) = lo;
    *reinterpret_cast<uint4*>(dst + (((p0 + 1) ^ (R & 15)) << 4)) = hi;
  };
  auto compute = [&](int r, int nkb, auto FULL_) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(FULL_)::value;
    const unsigned char* sl = smem + (r % D) * Cfg::SLOT;
    v2i braw[SWAVES];
    v2i araw[SWAVES][Cfg::TPW];
    v8bf abf[SWAVES][Cfg::TPW];
    float sbv[SWAVES], sav[SWAVES][2], sat[SWAVES][Cfg::TPW];
#pragma unroll
    for (int q = 0; q < SWAVES; ++q) {
      braw[q] = *reinterpret_cast<const v2i*>(sl + frag_off(16 * cs + (lane & 15), q));
#pragma unroll
      for (int t = 0; t < Cfg::TPW; ++t) {
        if constexpr (Cfg::A_SHARED) {
          const int row = 16 * tile_of(t) + (lane & 15);
          const unsigned char* ab = smem + Cfg::ABUF_OFF + (r & 1) * (32 * 512) + row * 512;
          abf[q][t] = *reinterpret_cast<const v8bf*>(ab + (((4 * q + (lane >> 4)) ^ (row & 15)) << 4));
        } else {
          araw[q][t] = *reinterpret_cast<const v2i*>(sl + Cfg::A_OFF + frag_off(16 * tile_of(t) + (lane & 15), q));
        }
      }
      const float* scr = reinterpret_cast<const float*>(sl + Cfg::SC_OFF + q * Cfg::REC);
      if constexpr (TG) {
#pragma unroll
        for (int t = 0; t < Cfg::TPW; ++t) sat[q][t] = scr[16 * tile_of(t) + (lane & 15)];
        sbv[q] = scr[(Cfg::TG_PACKED ? 32 : 64) + own_cb];
      } else {
        // the round record (wave 0's)
        const float* rec = reinterpret_cast<const float*>(sl + Cfg::SC_OFF);
        sav[q][0] = rec[q];
        sav[q][1] = rec[8 + q];
        sbv[q] = rec[16 + q * NCB + own_cb];
      }
    }
#pragma unroll
    for (int q = 0; q < SWAVES; ++q) {
      const v8bf bfrag = e4m3x8_to_bf16x8(braw[q]);
#pragma unroll
      for (int t = 0; t < Cfg::TPW; ++t) {
        const v8bf afrag = Cfg::A_SHARED ? abf[q][t] : e4m3x8_to_bf16x8(araw[q][t]);
        const v4f p = TG ? mfma_partial(bfrag, afrag) : mfma_partial(afrag, bfrag);
        const float sc = (TG ? sat[q][t] : sav[q][tile_of(t) >> 1]) * sbv[q];
        if (FULL || q < nkb) promote(acc[t], p, sc);
      }
    }
  };

  const int rounds = (KB + SWAVES - 1) / SWAVES;
  const int full_rounds = KB / SWAVES;
  if (KB > 0) {
#pragma unroll
    for (int d = 0; d < D - 1; ++d) issue(d);
  }
  for (int r = 0; r < rounds; ++r) {
    // this wave's round-r loads have landed: NCB + a_live + 1 loads per round
    constexpr int LB = (D - 2) * (NCB + Cfg::SCL);
    constexpr int LB0 = Cfg::ROUND_SC ? D - 2 : 0;  // wave 0's round records (wave 0 always loads A)
    if (a_live == 0) wait_vmcnt<LB>();
    else if (a_live == 1) {
      if (w == 0) wait_vmcnt<LB + LB0 + (D - 2)>();
      else wait_vmcnt<LB + (D - 2)>();
    } else {
      if (w == 0) wait_vmcnt<LB + LB0 + 2 * (D - 2)>();
      else wait_vmcnt<LB + 2 * (D - 2)>();
    }
    // the shared A area of round r - 2 is free: every wave finished that
    // round's compute before the previous barrier
    if constexpr (Cfg::A_SHARED) decode_own_a(r);
    lds_barrier();                     // ... and everyone else's; round r-1's slot is free
    issue(r + D - 1);                  // refill the slot that round r-1 used
    if (owns) {
      if (r < full_rounds) compute(r, SWAVES, std::true_type{});
      else compute(r, KB - r * SWAVES, std::false_type{});
    }
  }
  wait_vmcnt<0>();
  (void)n_slices;

#pragma unroll
  for (int t = 0; t < Cfg::TPW; ++t) {
    const int i = rg + t * Cfg::RG;
    if (owns && i < MT) {
      if constexpr (TG) {
        // lane holds row 16*i + (lane&15), columns cs*16 + 4*(lane>>4) + 0..3
        const int64_t row = i * 16 + (lane & 15);
        const int64_t col4 = n0 + cs * 16 + 4 * (lane >> 4);
        if (row < M) {
          const uint32_t lo = bf16_out(acc[t][0]) | (bf16_out(acc[t][1]) << 16);
          const uint32_t hi = bf16_out(acc[t][2]) | (bf16_out(acc[t][3]) << 16);
          *reinterpret_cast<uint2*>(c + row * N + col4) = make_uint2(lo, hi);
        }
      } else {
        const int col = (int)n0 + cs * 16 + (lane & 15);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int64_t row = i * 16 + 4 * (lane >> 4) + rr;
          if (row < M) c[row * N + col] = (uint16_t)bf16_out(acc[t][rr]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// small-M kernel, K-major weight, K-blocks split over the waves
// ------------------------------------------------------------------------------------
// When the workgroup's slice has fewer 16x16 output sub-tiles than waves,
// owning whole sub-tiles leaves most waves idle while the owners form eight K-blocks of
// partials per round.  Here every wave forms the partials of one K-block of the
// round for all sub-tiles (phase 1) and parks them in LDS; in the next round
// all 512 lanes promote them, each lane owning whole output elements and
// running their chain over the round's K-blocks in ascending order with the
// same fma(P, sa*sb, acc) as every other kernel (phase 2).  The partials are
// the same MFMA results, so every bit of C is unchanged.  Refills target the
// slot of two rounds back: phase 2 still reads the scale records of the
// previous round's slot.
template <int MT, int NCB, bool TG = false>
struct SmallMNtSplitCfg {
  static constexpr int W = 32 * NCB;
  static constexpr int CS = 2 * NCB;
  static constexpr int T = MT * CS;                   // output sub-tiles of the workgroup
  static constexpr int EPL = T * 256 / STHREADS;      // output elements per lane
  static constexpr int ACH = (MT + 1) / 2;
  static constexpr int A_OFF = W * 256;
  static constexpr int SC_OFF = A_OFF + 16 * MT * 256;  // the 16*MT A rows the fragments read
  static constexpr int REC = TG ? 512 : 256;
  static constexpr int SLOT = SC_OFF + SWAVES * REC;
  static constexpr int PB_BYTES = 2 * SWAVES * T * 1024;  // partials of two rounds
  static constexpr int D_FIT = (SMALL_LDS_BUDGET - PB_BYTES) / SLOT;
  static constexpr int D = D_FIT > 8 ? 8 : D_FIT;
  static constexpr int PB_OFF = D * SLOT;
  static constexpr int LDS = PB_OFF + PB_BYTES;
  static_assert(T * 256 % STHREADS == 0, "whole elements per lane");
  static_assert(D >= 3, "ring too shallow");
  static_assert(LDS <= SMALL_LDS_BUDGET, "LDS budget");
  static_assert((D - 3) * (NCB + ACH + (TG ? 2 : 1)) < 64, "vmcnt range");
  // 32x32 scales: wave 0 loads the whole round's scale record with one direct
  // load; SCL = scale loads per round of the other waves
  // token-group scales (at most 16 rows here): waves 0 and 1 load sa of rows
  // 0-7 and 8-15 for the round's eight K-blocks, wave 2 the sb entries, one
  // direct load each; RSW = waves that load a round record
  static constexpr bool ROUND_SC = true;
  static constexpr int SCL = 0;
  static constexpr int RSW = TG ? 3 : 1;
  static_assert(!TG || MT == 1, "token-group round records hold 16 rows");
};

template <int MT, int NCB, bool TG>
__global__ void __launch_bounds__(STHREADS) gemm_smallm_nt_split_kernel(const uint8_t* __restrict__ a,
                                                                        const float* __restrict__ sa,
                                                                        const uint8_t* __restrict__ bt,
                                                                        const float* __restrict__ sbt,
                                                                        uint16_t* __restrict__ c, int64_t M,
                                                                        int64_t N, int64_t K) {
  using Cfg = SmallMNtSplitCfg<MT, NCB, TG>;
  constexpr int D = Cfg::D, W = Cfg::W, CS = Cfg::CS, T = Cfg::T, EPL = Cfg::EPL;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int w = wave_id_uniform();
  const int KB = (int)(K >> 5);
  const int64_t n0 = (int64_t)blockIdx.x * W;
  const int cb0 = (int)(n0 >> 5);

  // ---- direct loads of round r (as in gemm_smallm_nt_kernel): weight pieces of
  // rows 4*(w*NCB+i).., A pieces of rows 4*(w+8*ch).. (only pieces with a row < M),
  // and the scale record of K-block 8r+w
  const int lp = lane & 15;
  const uint8_t* b_row[NCB];
  int b_g[NCB];
#pragma unroll
  for (int i = 0; i < NCB; ++i) {
    const int r = 4 * (w * NCB + i) + (lane >> 4);
    b_row[i] = bt + (n0 + r) * K;
    b_g[i] = lp ^ (r & 15);
  }
  const uint8_t* a_row[Cfg::ACH];
  int a_g[Cfg::ACH];
  int a_live = 0;
#pragma unroll
  for (int ch = 0; ch < Cfg::ACH; ++ch) {
    const int r = 4 * (w + 8 * ch) + (lane >> 4);
    const int64_t rr = r < M ? r : M - 1;
    a_row[ch] = a + rr * K;
    a_g[ch] = lp ^ (r & 15);
    a_live += 4 * (w + 8 * ch) < M ? 1 : 0;
  }
  const int nrb = (int)((M + 31) >> 5);
  // round record (wave 0), as in gemm_smallm_nt_kernel: lane l < 16 = sa of
  // row-block min(l >> 3, nrb-1) at K-block 8r + (l & 7); lane 16 + q*NCB + c =
  // sbt of column block cb0 + c at K-block 8r + q; K-blocks clamped to the last
  const int rs_l = lane < 16 ? lane : (lane - 16 < 8 * NCB ? lane - 16 : 8 * NCB - 1);
  const int rs_q = lane < 16 ? (rs_l & 7) : rs_l / NCB;
  const float* const rs_src = lane < 16 ? sa + (int64_t)((lane >> 3) < nrb ? (lane >> 3) : nrb - 1) * KB
                                        : sbt + (int64_t)(cb0 + rs_l % NCB) * KB;
  // token-group round records: wave w < 2, lane l = sa of row 8w + (l >> 3)
  // (clamped to M-1) at K-block 8r + (l & 7); wave 2, lane l = sbt of column
  // block cb0 + c at K-block 8r + q for l = q * NCB + c (lanes past 8 * NCB
  // repeat the last entry); both step 1 per K-block
  const int tg_l = lane < 8 * NCB ? lane : 8 * NCB - 1;
  const int tg_q = w < 2 ? (lane & 7) : tg_l / NCB;
  const int tg_row = 8 * w + (lane >> 3);
  const float* const tg_rs_src = w < 2 ? sa + (int64_t)(tg_row < M ? tg_row : M - 1) * KB
                                       : sbt + (int64_t)(cb0 + tg_l % NCB) * KB;
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  const uint32_t ring = (uint32_t)(uintptr_t)((lds_u8*)smem);

  auto koff = [&](int r, int g) __attribute__((always_inline)) -> int64_t {
    int kb = r * SWAVES + (g >> 1);
    kb = kb < KB ? kb : KB - 1;
    return (int64_t)kb * 32 + (g & 1) * 16;
  };
  auto issue = [&](int r) __attribute__((always_inline)) {
    const uint32_t sl = ring + (r % D) * Cfg::SLOT;
#pragma unroll
    for (int i = 0; i < NCB; ++i) dma16(b_row[i] + koff(r, b_g[i]), sl + (w * NCB + i) * 1024);
#pragma unroll
    for (int ch = 0; ch < Cfg::ACH; ++ch)
      if (ch < a_live) dma16(a_row[ch] + koff(r, a_g[ch]), sl + Cfg::A_OFF + (w + 8 * ch) * 1024);
    int kc = r * SWAVES + w;
    kc = kc < KB ? kc : KB - 1;
    if constexpr (TG) {
      if (w < 3) {
        int kr = r * SWAVES + tg_q;
        kr = kr < KB ? kr : KB - 1;
        dma4(tg_rs_src + kr, sl + Cfg::SC_OFF + w * Cfg::REC);
      }
    } else {
      if (w == 0) {
        int kr = r * SWAVES + rs_q;
        kr = kr < KB ? kr : KB - 1;
        dma4(rs_src + kr, sl + Cfg::SC_OFF);
      }
    }
  };

  const int fr_half = ((lane >> 4) & 1) * 8, fr_hi = lane >> 5;
  auto frag_off = [&](int row, int q) __attribute__((always_inline)) {
    return row * 256 + 16 * ((2 * q + fr_hi) ^ (lane & 15)) + fr_half;
  };

  // phase 1: this wave's K-block (q = w) of round r, every sub-tile t = i*CS + cs
  auto phase1 = [&](int r) __attribute__((always_inline)) {
    const unsigned char* sl = smem + (r % D) * Cfg::SLOT;
    v2i braw[CS], araw[MT];
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) braw[cs] = *reinterpret_cast<const v2i*>(sl + frag_off(16 * cs + (lane & 15), w));
#pragma unroll
    for (int i = 0; i < MT; ++i)
      araw[i] = *reinterpret_cast<const v2i*>(sl + Cfg::A_OFF + frag_off(16 * i + (lane & 15), w));
    v8bf bf[CS], af[MT];
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) bf[cs] = e4m3x8_to_bf16x8(braw[cs]);
#pragma unroll
    for (int i = 0; i < MT; ++i) af[i] = e4m3x8_to_bf16x8(araw[i]);
    unsigned char* pb = smem + Cfg::PB_OFF + ((r & 1) * SWAVES + w) * T * 1024;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) {
        const v4f p = TG ? mfma_partial(bf[cs], af[i]) : mfma_partial(af[i], bf[cs]);
        *reinterpret_cast<v4f*>(pb + (i * CS + cs) * 1024 + lane * 16) = p;
      }
  };

  // phase 2: lane G = 64w + lane owns elements e = G + 512j of the workgroup's
  // T*256 (sub-tile e >> 8, MFMA output slot e & 255)
  const int G = w * 64 + lane;
  float acc[EPL];
  int e_row[EPL], e_col[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    acc[j] = 0.0f;
    const int e = G + STHREADS * j, t = e >> 8, f = e & 255;
    const int l = f >> 2, i4 = f & 3;
    const int row_in = TG ? (l & 15) : 4 * (l >> 4) + i4;
    const int col_in = TG ? 4 * (l >> 4) + i4 : (l & 15);
    e_row[j] = 16 * (t / CS) + row_in;
    e_col[j] = 16 * (t % CS) + col_in;
  }
  auto phase2 = [&](int r, int nkb) __attribute__((always_inline)) {
    const unsigned char* sl = smem + (r % D) * Cfg::SLOT;
    const unsigned char* pb = smem + Cfg::PB_OFF + (r & 1) * SWAVES * T * 1024;
#pragma unroll
    for (int q = 0; q < SWAVES; ++q) {
      if (q < nkb) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
          const int e = G + STHREADS * j;
          const float p = *reinterpret_cast<const float*>(pb + (q * T + (e >> 8)) * 1024 + (e & 255) * 4);
          const int own_cb = e_col[j] >> 5;
          // round records: 32x32 scales in wave 0's; token groups: sa of row r
          // in wave (r >> 3)'s at lane (r & 7) * 8 + q, sb in wave 2's
          const float* rec = reinterpret_cast<const float*>(sl + Cfg::SC_OFF);
          const float sc = TG ? rec[(e_row[j] >> 3) * (Cfg::REC / 4) + (e_row[j] & 7) * 8 + q] *
                                    rec[2 * (Cfg::REC / 4) + q * NCB + own_cb]
                              : rec[8 * (e_row[j] >> 5) + q] * rec[16 + q * NCB + own_cb];
          acc[j] = __builtin_fmaf(p, sc, acc[j]);
        }
      }
    }
  };

  const int rounds = (KB + SWAVES - 1) / SWAVES;
  if (KB > 0) {
#pragma unroll
    for (int d = 0; d < D - 2; ++d) issue(d);
  }
  for (int r = 0; r < rounds; ++r) {
    // this wave's round-r loads have landed: NCB + a_live + scale loads per round, D - 3 rounds may be pending
    constexpr int LB = (D - 3) * (NCB + Cfg::SCL);
    // round records: waves below RSW load one per round
    constexpr int LB0 = D - 3;
    const bool rs = w < Cfg::RSW;
    if (a_live == 0) {
      if (rs) wait_vmcnt<LB + LB0>();
      else wait_vmcnt<LB>();
    } else if (a_live == 1) {
      if (rs) wait_vmcnt<LB + LB0 + (D - 3)>();
      else wait_vmcnt<LB + (D - 3)>();
    } else {
      if (rs) wait_vmcnt<LB + LB0 + 2 * (D - 3)>();
      else wait_vmcnt<LB + 2 * (D - 3)>();
    }
    lds_barrier();   // round r visible; round r-1's partials visible; round r-2's slot free
    issue(r + D - 2);
    // Promotion of round r-1 first: its partial and scale reads then precede
    // this round's partial stores in program order, so the compiler may
    // overlap the two chains (phase 1 writes the other partial buffer, and
    // the refill above targets the slot of round r-2).  Measured 24.8 against
    // 25.3 us at N = K = 8192, M = 1.
    if (r > 0) phase2(r - 1, SWAVES);   // only the last round can be partial
    phase1(r);
  }
  if (rounds > 0) {
    lds_barrier();
    phase2(rounds - 1, KB - (rounds - 1) * SWAVES);
  }
  wait_vmcnt<0>();

#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int64_t row = e_row[j];
    if (row < M) c[row * N + n0 + e_col[j]] = (uint16_t)bf16_out(acc[j]);
  }
}

// ------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------
// act_tg: A's scales are per token group, [M, K/32], instead of [ceil(M/32), K/32].
template <bool BT, bool TG>
static void launch_tile_t(const void* a, const float* sa, const void* b, const float* sb, void* c, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream) {
  const int64_t tiles_m = (M + TBM - 1) / TBM, tiles_n = (N + TBN - 1) / TBN;
  const int64_t n_tiles = tiles_m * tiles_n;
  const int remap = (n_tiles % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((gemm_tile_kernel<BT, TG>), dim3((unsigned)n_tiles), dim3(TTHREADS), TILE_LDS_BYTES, stream,
                     (const uint8_t*)a, sa, (const uint8_t*)b, sb, (uint16_t*)c, M, N, K, tiles_m, tiles_n, remap);
}

hipError_t launch_gemm_tile(const void* a, const float* sa, const void* b, const float* sb, void* c, int64_t M,
                            int64_t N, int64_t K, bool k_major_b, bool act_tg, hipStream_t stream) {
  if (k_major_b) {
    if (act_tg) launch_tile_t<true, true>(a, sa, b, sb, c, M, N, K, stream);
    else launch_tile_t<true, false>(a, sa, b, sb, c, M, N, K, stream);
  } else {
    if (act_tg) launch_tile_t<false, true>(a, sa, b, sb, c, M, N, K, stream);
    else launch_tile_t<false, false>(a, sa, b, sb, c, M, N, K, stream);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const void* a, const float* sa, const void* b, const float* sb,
                               const int32_t* offsets, int G, void* c, int64_t M_total, int64_t N, int64_t K,
                               bool k_major_b, hipStream_t stream) {
  const int64_t tiles_n = (N + TBN - 1) / TBN;
  // an upper bound on the tile count: the sum over groups of ceil(M_g / 256)
  const int64_t grid = (M_total / TBM + G) * tiles_n;
  if (k_major_b)
    hipLaunchKernelGGL(gemm_grouped_kernel<true>, dim3((unsigned)grid), dim3(TTHREADS), TILE_LDS_BYTES, stream,
                       (const uint8_t*)a, sa, (const uint8_t*)b, sb, offsets, G, (uint16_t*)c, M_total, N, K, tiles_n);
  else
    hipLaunchKernelGGL(gemm_grouped_kernel<false>, dim3((unsigned)grid), dim3(TTHREADS), TILE_LDS_BYTES, stream,
                       (const uint8_t*)a, sa, (const uint8_t*)b, sb, offsets, G, (uint16_t*)c, M_total, N, K, tiles_n);
  return hipGetLastError();
}

// Column-slice width for the small-M kernel, [K, N] weight: 128-byte slices
// read whole cache lines of B, but the grid must still cover most of the 256 CUs.
int smallm_ncb(int64_t N) {
  if (N % 128 == 0 && N / 128 >= 192) return 4;
  if (N % 64 == 0 && N / 64 >= 192) return 2;
  return 1;
}

// K-major weight: every slice streams whole rows whatever its width, so the
// width only balances the grid over the 256 CUs (the fraction of the last wave
// of workgroups that is busy); ties go to the wider slice.
int smallm_nt_ncb(int64_t N) {
  int best = 1;
  double best_fill = -1.0;
  for (int ncb : {4, 2, 1}) {
    const int64_t w = 32 * ncb;
    if (N % w) continue;
    const int64_t g = N / w;
    const double fill = (double)g / (double)(((g + 255) / 256) * 256);
    if (fill > best_fill + 1e-9) {
      best_fill = fill;
      best = ncb;
    }
  }
  return best;
}

// 32-column K-major slices with at most 16 rows (two sub-tiles, six of eight
// waves idle in gemm_smallm_nt_kernel) use the split kernel: 25.3 against
// 27.3 us at N = K = 8192.  With four sub-tiles the parked partials leave
// room for only four or five ring slots, which costs more than the idle
// waves (35.8 against 29.8 us at M = 32).
template <int MT, int NCB>
constexpr bool kNtSplit = MT * 2 * NCB <= 2;

template <int MT, int NCB, bool NT, bool TG>
static void launch_smallm_t(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, uint16_t* c,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if constexpr (NT && kNtSplit<MT, NCB>) {
    using Cfg = SmallMNtSplitCfg<MT, NCB, TG>;
    hipLaunchKernelGGL((gemm_smallm_nt_split_kernel<MT, NCB, TG>), dim3((unsigned)(N / Cfg::W)), dim3(STHREADS),
                       Cfg::LDS, stream, a, sa, b, sb, c, M, N, K);
  } else if constexpr (NT) {
    using Cfg = SmallMNtCfg<MT, NCB, TG>;
    hipLaunchKernelGGL((gemm_smallm_nt_kernel<MT, NCB, TG>), dim3((unsigned)(N / Cfg::W)), dim3(STHREADS), Cfg::LDS,
                       stream, a, sa, b, sb, c, M, N, K);
  } else {
    using Cfg = SmallMCfg<MT, NCB, TG>;
    hipLaunchKernelGGL((gemm_smallm_kernel<MT, NCB, TG>), dim3((unsigned)(N / Cfg::W)), dim3(STHREADS), Cfg::LDS,
                       stream, a, sa, b, sb, c, M, N, K);
  }
}

template <int NCB, bool NT, bool TG>
static void launch_smallm_n(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, uint16_t* c,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  switch ((int)((M + 15) / 16)) {
    case 1: launch_smallm_t<1, NCB, NT, TG>(a, sa, b, sb, c, M, N, K, stream); break;
    case 2: launch_smallm_t<2, NCB, NT, TG>(a, sa, b, sb, c, M, N, K, stream); break;
    case 3: launch_smallm_t<3, NCB, NT, TG>(a, sa, b, sb, c, M, N, K, stream); break;
    default: launch_smallm_t<4, NCB, NT, TG>(a, sa, b, sb, c, M, N, K, stream); break;
  }
}

template <bool NT, bool TG>
static void launch_smallm_l(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, uint16_t* c,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  switch (NT ? smallm_nt_ncb(N) : smallm_ncb(N)) {
    case 4: launch_smallm_n<4, NT, TG>(a, sa, b, sb, c, M, N, K, stream); break;
    case 2: launch_smallm_n<2, NT, TG>(a, sa, b, sb, c, M, N, K, stream); break;
    default: launch_smallm_n<1, NT, TG>(a, sa, b, sb, c, M, N, K, stream); break;
  }
}

hipError_t launch_gemm_smallm(const void* a, const float* sa, const void* b, const float* sb, void* c, int64_t M,
                              int64_t N, int64_t K, bool k_major_b, bool act_tg, hipStream_t stream) {
  const uint8_t* a8 = (const uint8_t*)a;
  const uint8_t* b8 = (const uint8_t*)b;
  uint16_t* c16 = (uint16_t*)c;
  if (k_major_b) {
    if (act_tg) launch_smallm_l<true, true>(a8, sa, b8, sb, c16, M, N, K, stream);
    else launch_smallm_l<true, false>(a8, sa, b8, sb, c16, M, N, K, stream);
  } else {
    if (act_tg) launch_smallm_l<false, true>(a8, sa, b8, sb, c16, M, N, K, stream);
    else launch_smallm_l<false, false>(a8, sa, b8, sb, c16, M, N, K, stream);
  }
  return hipGetLastError();
}

template <int MT, int NCB, bool TG>
static hipError_t set_smallm_attr() {
  hipError_t e = hipFuncSetAttribute((const void*)gemm_smallm_kernel<MT, NCB, TG>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, SmallMCfg<MT, NCB, TG>::LDS);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)gemm_smallm_nt_kernel<MT, NCB, TG>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, SmallMNtCfg<MT, NCB, TG>::LDS);
  if (e != hipSuccess) return e;
  if constexpr (kNtSplit<MT, NCB>)
    e = hipFuncSetAttribute((const void*)gemm_smallm_nt_split_kernel<MT, NCB, TG>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, SmallMNtSplitCfg<MT, NCB, TG>::LDS);
  return e;
}

template <int NCB, bool TG>
static hipError_t set_smallm_attrs() {
  hipError_t e;
  if ((e = set_smallm_attr<1, NCB, TG>()) != hipSuccess) return e;
  if ((e = set_smallm_attr<2, NCB, TG>()) != hipSuccess) return e;
  if ((e = set_smallm_attr<3, NCB, TG>()) != hipSuccess) return e;
  return set_smallm_attr<4, NCB, TG>();
}

hipError_t set_gemm_attributes() {
  const void* tiles[6] = {(const void*)gemm_tile_kernel<false, false>, (const void*)gemm_tile_kernel<true, false>,
                          (const void*)gemm_tile_kernel<false, true>,  (const void*)gemm_tile_kernel<true, true>,
                          (const void*)gemm_grouped_kernel<false>,     (const void*)gemm_grouped_kernel<true>};
  hipError_t e;
  for (const void* f : tiles)
    if ((e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, TILE_LDS_BYTES)) != hipSuccess)
      return e;
  if ((e = set_smallm_attrs<1, false>()) != hipSuccess) return e;
  if ((e = set_smallm_attrs<2, false>()) != hipSuccess) return e;
  if ((e = set_smallm_attrs<4, false>()) != hipSuccess) return e;
  if ((e = set_smallm_attrs<1, true>()) != hipSuccess) return e;
  if ((e = set_smallm_attrs<2, true>()) != hipSuccess) return e;
  return set_smallm_attrs<4, true>();
}

}  // namespace fp8bs
