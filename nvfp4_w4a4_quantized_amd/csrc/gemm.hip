// Block-scaled W4A4 GEMM kernels for gfx950.
//
// Operands stay packed (4-bit codes + E4M3 block scales) in HBM and LDS.  Each lane
// decodes its MFMA operand in registers: 8 codes (one dword) -> f16 e2m1 values by the
// hardware fp4 conversion, times the block scale as f16 (exact: the product has <= 6
// significant bits and lies in [2^-10, 2688]).  f16 x f16 products are exact in
// fp32; MFMA accumulates in fp32.  The epilogue multiplies column n by
// g_a * g_w[segment(n)] (the per-segment global-scale repair for fused GEMMs over
// per-module-calibrated weights: "Why Gated DeltaNet Survives 4-Bit Quantization"
// review page, strengths paragraph / the paper's section 6) and optionally applies
// the GDN gates of Eq. 1 (same page, mechanism step 2).
//
// K-permutation.  A lane loads 16 contiguous bytes (32 elements) of its row; MFMA
// step t uses dword t of them.  Both operands use the same permutation of k, so the
// sum over k is unchanged, and every 8-element group a lane feeds to one MFMA lies
// inside one 16-element scale block.
#include "kernel_common.hpp"

namespace nvfp4 {

namespace {

// ---------------------------------------------------------------------------------
// Tiled GEMM: 128 x 128 output tile per workgroup, BK = 64, 4 waves of 64 x 64,
// MFMA 32x32x16 f16.  Packed tiles are staged through LDS (codes 4 KiB + scales
// 512 B per operand per K step) with a register prefetch of the next step.
// ---------------------------------------------------------------------------------
constexpr int TBM = 128, TBN = 128, TBK = 64;

struct TileRegs {
  u32x4 ca, cw;     // 16 bytes of codes for A and W
  uint32_t sc;      // 4 scale bytes (A for threads < 128, W otherwise)
};

template <bool ALIGNED>
__device__ __forceinline__ u32x4 load_codes16(const uint8_t* base, int64_t row, int64_t rows, int64_t K,
                                              int64_t k0, int h) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if (row >= rows) return r;
  const int64_t kk = k0 + 32 * h;             // first element of this half
  const uint8_t* p = base + row * (K >> 1) + (kk >> 1);
  if constexpr (ALIGNED) {
    r = *reinterpret_cast<const u32x4*>(p);
  } else {
    // K % 64 != 0: load 8 bytes (16 elements) at a time, only inside the row
    if (kk < K) {
      const uint2 lo = *reinterpret_cast<const uint2*>(p);
      r[0] = lo.x; r[1] = lo.y;
    }
    if (kk + 16 < K) {
      const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
      r[2] = hi.x; r[3] = hi.y;
    }
  }
  return r;
}

template <bool ALIGNED>
__device__ __forceinline__ uint32_t load_scales4(const uint8_t* base, int64_t row, int64_t rows, int64_t K,
                                                 int64_t k0) {
  if (row >= rows) return 0u;
  const int64_t kb = K >> 4;
  const uint8_t* p = base + row * kb + (k0 >> 4);
  if constexpr (ALIGNED) {
    return *reinterpret_cast<const uint32_t*>(p);
  } else {
    uint32_t r = 0;
    for (int j = 0; j < 4; ++j)
      if ((k0 >> 4) + j < kb) r |= (uint32_t)p[j] << (8 * j);
    return r;
  }
}

template <bool ALIGNED, int EPI, bool RC>
__global__ __launch_bounds__(256) void k_gemm_tiled(GemmArgs a) {
  __shared__ u32x4 lds_ca[2][TBM];
  __shared__ u32x4 lds_cw[2][TBN];
  __shared__ uint32_t lds_sa[TBM];
  __shared__ uint32_t lds_sw[TBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, li = lane & 31;

  // tile order: groups of 8 row-tiles sweep the column tiles (L2 reuse of W)
  const int64_t tiles_m = (a.M + TBM - 1) / TBM;
  const int64_t tiles_n = (a.N + TBN - 1) / TBN;
  const int64_t pid = blockIdx.x;
  const int64_t group = 8;
  const int64_t per_group = group * tiles_n;
  const int64_t gid = pid / per_group;
  const int64_t first_m = gid * group;
  const int64_t gsize = (tiles_m - first_m) < group ? (tiles_m - first_m) : group;
  const int64_t bm = first_m + (pid % per_group) % gsize;
  const int64_t bn = (pid % per_group) / gsize;
  const int64_t m0 = bm * TBM, n0 = bn * TBN;

  // loader roles: thread -> (row, half) for codes; threads < 128 load A scales, others W
  const int lrow = tid >> 1, lh = tid & 1;
  const int srow = tid & 127;
  const bool s_is_a = tid < 128;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto gload = [&](int64_t k0) {
    TileRegs t;
    t.ca = load_codes16<ALIGNED>(a.a_codes, m0 + lrow, a.M, a.K, k0, lh);
    t.cw = load_codes16<ALIGNED>(a.w_codes, n0 + lrow, a.N, a.K, k0, lh);
    t.sc = s_is_a ? load_scales4<ALIGNED>(a.a_scales, m0 + srow, a.M, a.K, k0)
                  : load_scales4<ALIGNED>(a.w_scales, n0 + srow, a.N, a.K, k0);
    return t;
  };

  TileRegs cur = gload(0);
  for (int64_t k0 = 0; k0 < a.K; k0 += TBK) {
    lds_ca[lh][lrow] = cur.ca;
    lds_cw[lh][lrow] = cur.cw;
    if (s_is_a) lds_sa[srow] = cur.sc; else lds_sw[srow] = cur.sc;
    __syncthreads();
    if (k0 + TBK < a.K) cur = gload(k0 + TBK);

    f16x8 A[2][4], B[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + i * 32 + li;
      const u32x4 c = lds_ca[h][r];
      const uint32_t s = lds_sa[r] >> (16 * h);
      const f16x2 s0 = scale_f16x2(s & 0xFFu), s1 = scale_f16x2((s >> 8) & 0xFFu);
      A[i][0] = decode8_f16(c[0], s0);
      A[i][1] = decode8_f16(c[1], s0);
      A[i][2] = decode8_f16(c[2], s1);
      A[i][3] = decode8_f16(c[3], s1);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wn * 64 + j * 32 + li;
      const u32x4 c = lds_cw[h][r];
      const uint32_t s = lds_sw[r] >> (16 * h);
      const f16x2 s0 = scale_f16x2(s & 0xFFu), s1 = scale_f16x2((s >> 8) & 0xFFu);
      B[j][0] = decode8_f16(c[0], s0);
      B[j][1] = decode8_f16(c[1], s0);
      B[j][2] = decode8_f16(c[2], s1);
      B[j][3] = decode8_f16(c[3], s1);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i][t], B[j][t], acc[i][j], 0, 0, 0);
    __syncthreads();
  }

  const float ga = *a.a_gscale;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wn * 64 + j * 32 + li;
    const bool n_ok = n < a.N;
    float alpha = n_ok ? col_alpha<EPI>(a, n, ga) : 0.0f;
    if constexpr (RC) alpha = n_ok ? alpha * a.col_scale[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if constexpr (RC) {
          if (n_ok && m < a.M) store_out_rc<EPI>(a, m, n, acc[i][j][r], alpha, a.row_scale[m]);
        } else {
          if (n_ok && m < a.M) store_out<EPI>(a, m, n, acc[i][j][r], alpha);
        }
      }
  }
}

// ---------------------------------------------------------------------------------
// Large-tile GEMM for prefill shapes: 256 x 256 output tile per workgroup, BK = 64,
// 4 waves of 128 x 128 (4 x 4 MFMA 32x32x16 f16, 256 fp32 accumulators per lane in
// AGPRs, so one wave per SIMD).  Decode work per wave grows with (128 + 128) while
// MFMA work grows with 128 x 128.
//
// Data movement: packed tiles (codes 16 KiB + scales 2 KiB per K step) go from HBM
// straight into a 4-stage LDS ring with gfx950's direct-to-LDS loads (no staging
// registers, no ds_write); the loads of K step k+3 are issued while step k computes.
// Before the barrier that publishes stage k+1 each wave waits only for its own loads
// of that stage (vmcnt), so two later stages stay in flight.
//
// Software pipeline inside a K step (4 MFMA steps of K = 16): while the 16 MFMAs of
// step t run, the lane decodes the operands of step t+1 (interleaved 1 MFMA : 4 VALU
// by sched_group_barrier).  The barrier sits before the last MFMA step, so the next
// K step's LDS reads and its step-0 decode run under those MFMAs.
// Requires K % 64 == 0 and K >= 192 (three K steps).
// ---------------------------------------------------------------------------------
constexpr int GBM = 256, GBN = 256, GBK = 64;

// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs (each with its
// own L2), so workgroup id p runs on XCD p % 8.  When the tile count divides by 8,
// XCD x is given the contiguous logical tiles [x*T/8, (x+1)*T/8); logical tiles are
// ordered in groups of 4 row tiles sweeping the column tiles.  The ~32 workgroups
// an XCD runs at once then cover a 4 x 8 block of tiles: 12 operand tiles per K
// step come through its L2 instead of 33 with a plain row-group order.
__device__ __forceinline__ void big_tile_of(int64_t M, int64_t N, int64_t pid, int64_t* bm, int64_t* bn) {
  const int64_t tiles_m = (M + GBM - 1) / GBM;
  const int64_t tiles_n = (N + GBN - 1) / GBN;
  const int64_t num = tiles_m * tiles_n;
  const int64_t logical = (num % 8 == 0) ? (pid % 8) * (num / 8) + pid / 8 : pid;
  const int64_t group = 4;
  const int64_t per_group = group * tiles_n;
  const int64_t first_m = (logical / per_group) * group;
  const int64_t gsize = (tiles_m - first_m) < group ? (tiles_m - first_m) : group;
  *bm = first_m + (logical % per_group) % gsize;
  *bn = (logical % per_group) / gsize;
}
// Direct-to-LDS buffer loads: lane l lands at lds + size * l (the LDS address
// is wave-uniform, set in M0); vector offset per lane, scalar offset per wave.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}
constexpr int GST = 4;                                  // LDS stages
constexpr int ST_A = 0, ST_W = 8192, ST_SA = 16384, ST_SW = 17408, ST_BYTES = 18432;

template <int EPI, bool RC>
__global__ __launch_bounds__(256, 1) void k_gemm_big(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[GST * ST_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform values through readfirstlane: the compiler keeps what derives from
  // them (LDS bases, M0) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, li = lane & 31;

  int64_t bm, bn;
  big_tile_of(a.M, a.N, blockIdx.x, &bm, &bn);
  const int64_t m0 = bm * GBM, n0 = bn * GBN;
  const int64_t K = a.K;
  const int64_t kh = K >> 1, kb = K >> 4;

  // LDS stage layout: codes [row][32 B] (both halves of the row's 64 elements), the
  // two 16-byte halves of row r stored in swapped order when bit 2 xor bit 3 of r is
  // set, which makes the per-lane 16-byte reads below conflict-free; scales [row][4 B].
  // Load roles (per wave, per K step): 2 x 32 rows of A codes and of W codes (lanes
  // 2j and 2j+1 fetch the two halves of one row: 32 contiguous bytes), 64 rows of A
  // and of W scales.  Rows past M or N are clamped to the last row (in bounds; their
  // outputs are never stored).
  // Global addresses: a uniform base that advances with k (scalar registers) plus a
  // fixed 32-bit offset per lane (each packed operand is < 2^31 bytes, checked on the
  // host), so a load costs no vector address arithmetic.
  uint32_t oa_c[2], ow_c[2];
  uint32_t lo_c[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r0 = 32 * (2 * wave + q);
    const int row = r0 + (lane >> 1);
    const int hl = (lane & 1) ^ (((row >> 2) ^ (row >> 3)) & 1);      // logical half of this slot
    const int64_t ra = min<int64_t>(m0 + row, a.M - 1);
    const int64_t rw = min<int64_t>(n0 + row, a.N - 1);
    oa_c[q] = (uint32_t)(ra * kh + 16 * hl);
    ow_c[q] = (uint32_t)(rw * kh + 16 * hl);
    lo_c[q] = (uint32_t)(r0 * 32);
  }
  const uint32_t oa_s = (uint32_t)(min<int64_t>(m0 + 64 * wave + lane, a.M - 1) * kb);
  const uint32_t ow_s = (uint32_t)(min<int64_t>(n0 + 64 * wave + lane, a.N - 1) * kb);
  const uint32_t lo_s = (uint32_t)(64 * wave * 4);
  // buffer descriptors of the four packed operands (size = byte extent)
  const __amdgpu_buffer_rsrc_t ra_c = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.a_codes), (short)0,
                                                                        (int)(a.M * kh), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw_c = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.w_codes), (short)0,
                                                                        (int)(a.N * kh), 0x00020000);
  const __amdgpu_buffer_rsrc_t ra_s = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.a_scales), (short)0,
                                                                        (int)(a.M * kb), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw_s = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.w_scales), (short)0,
                                                                        (int)(a.N * kb), 0x00020000);
  auto issue = [&](int st, int64_t k0) {
    uint8_t* base = smem + st * ST_BYTES;
    const int kc = (int)(k0 >> 1), ks = (int)(k0 >> 4);          // wave-uniform offsets
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      buffer_load_lds16(ra_c, base + ST_A + lo_c[q], oa_c[q], kc);
      buffer_load_lds16(rw_c, base + ST_W + lo_c[q], ow_c[q], kc);
    }
    buffer_load_lds4(ra_s, base + ST_SA + lo_s, oa_s, ks);
    buffer_load_lds4(rw_s, base + ST_SW + lo_s, ow_s, ks);
  };

  // LDS read addresses: a per-lane base (computed once) plus the stage offset; the row
  // block i adds an immediate.  Row r = w*128 + i*32 + li: bits 2 and 3 of r (the
  // half swap) are those of li.
  const int swz = (li >> 2 ^ li >> 3) & 1;
  const uint32_t la_c = (uint32_t)(ST_A + (wm * 128 + li) * 32 + 16 * (h ^ swz));
  const uint32_t lw_c = (uint32_t)(ST_W + (wn * 128 + li) * 32 + 16 * (h ^ swz));
  const uint32_t la_s = (uint32_t)(ST_SA + (wm * 128 + li) * 4 + 2 * h);
  const uint32_t lw_s = (uint32_t)(ST_SW + (wn * 128 + li) * 4 + 2 * h);
  u32x4 ca[4], cw[4];          // packed codes of this lane's rows for the current K step
  f16x2 pa[4], pw[4];          // scale pairs {block 2h, block 2h+1}
  auto lread = [&](int st) {
    const uint8_t* base = smem + st * ST_BYTES;
    const uint8_t* pac = base + la_c;
    const uint8_t* pwc = base + lw_c;
    const uint8_t* pas = base + la_s;
    const uint8_t* pws = base + lw_s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ca[i] = *reinterpret_cast<const u32x4*>(pac + i * 1024);
      pa[i] = scale_pair_f16(*reinterpret_cast<const uint16_t*>(pas + i * 128));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cw[j] = *reinterpret_cast<const u32x4*>(pwc + j * 1024);
      pw[j] = scale_pair_f16(*reinterpret_cast<const uint16_t*>(pws + j * 128));
    }
  };
  f16x8 A0[4], B0[4], A1[4], B1[4];
  auto decode = [&](int t, f16x8 A[4], f16x8 B[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) A[i] = decode8_f16(ca[i][t], bcast(pa[i], t >> 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) B[j] = decode8_f16(cw[j][t], bcast(pw[j], t >> 1));
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto mfma_step = [&](const f16x8 A[4], const f16x8 B[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[j], acc[i][j], 0, 0, 0);
  };

  // One K step.  LOAD: issue the loads of tile k+3; NEXT: publish and read tile k+1
  // during the last MFMA step; VM: loads allowed in flight when tile k+1 is needed.
  const int64_t nk = K / GBK;
  auto kstep = [&]<bool LOAD, bool NEXT, int VM>(int64_t kt) {
    // step 0 MFMAs | decode step 1, loads of tile k+3
    mfma_step(A0, B0);
    decode(1, A1, B1);
    if constexpr (LOAD) {
      issue((int)((kt + 3) & 3), (kt + 3) * GBK);
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      SCHED_MFMA_VALU(10, 4)
    } else {
      SCHED_MFMA_VALU(16, 4)
    }
    // step 1 MFMAs | decode step 2
    mfma_step(A1, B1);
    decode(2, A0, B0);
    SCHED_MFMA_VALU(16, 4)
    // step 2 MFMAs | decode step 3
    mfma_step(A0, B0);
    decode(3, A1, B1);
    SCHED_MFMA_VALU(16, 4)
    if constexpr (NEXT) {
      wait_vmcnt<VM>();                 // this wave's loads of tile k+1 have landed
      wg_barrier();                     // ... and every other wave's
      lread((int)((kt + 1) & 3));
      mfma_step(A1, B1);
      decode(0, A0, B0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      SCHED_MFMA_VALU(12, 6)
    } else {
      mfma_step(A1, B1);
    }
  };

  issue(0, 0);
  issue(1, GBK);
  issue(2, 2 * GBK);
  wait_vmcnt<12>();
  wg_barrier();
  lread(0);
  decode(0, A0, B0);
  int64_t kt = 0;
  for (; kt + 3 < nk; ++kt) kstep.template operator()<true, true, 12>(kt);
  kstep.template operator()<false, true, 6>(kt);       // kt = nk - 3
  ++kt;
  kstep.template operator()<false, true, 0>(kt);       // kt = nk - 2
  ++kt;
  kstep.template operator()<false, false, 0>(kt);      // kt = nk - 1

  // Epilogue.  The four column scales are loaded together (no load waits for
  // another).  Interior tiles, which are all tiles when M and N are multiples of 256,
  // store without per-element bounds checks through a buffer descriptor of y: the
  // lane's part of the address is one VGPR offset fixed for the whole epilogue and the
  // rest (row block, row, column block) is a wave-uniform SGPR offset, so a store costs
  // no address arithmetic.  The byte extent of y must be < 2^32 (checked here); it is
  // also the descriptor's size, past which the hardware drops stores.  The stores are
  // non-temporal (cache policy nt): the output (268 MB at 8192 x 16384 bf16) does not
  // fit the caches anyway, and kept out of them it leaves the operand tiles that later
  // workgroups re-read in place (1.2% faster at 8192 x 16384 x 5120).
  // bf16 output is stored as 32-bit pairs of adjacent columns: rows 2p and 2p+1 of a
  // lane's column are converted together, the pair is swapped with the neighbouring
  // lane (DPP), and v_perm assembles [row 2p: columns c, c+1] on even lanes and
  // [row 2p+1: columns c-1, c] on odd lanes.
  const float ga = *a.a_gscale;
  float alpha[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 128 + j * 32 + li;
    alpha[j] = col_alpha<EPI>(a, min<int64_t>(n, a.N - 1), ga);
    if constexpr (RC) alpha[j] = alpha[j] * a.col_scale[min<int64_t>(n, a.N - 1)];
  }
  static_assert(EPI != EPI_GATE, "the gate epilogue runs in the 128x128-tile kernel");
  constexpr int ESZ = (EPI == EPI_BF16) ? 2 : 4;
  const int64_t extent = ((a.M - 1) * a.ldy + a.N) * ESZ;
  if constexpr (RC) {
    // With per-row factors the epilogue goes row block by row block, holding the 16 row
    // factors of one block at a time (all 64 in registers at once spilled to scratch):
    // y = (acc * fp32(alpha_n * col_n)) * row_m, each product rounded once.
    auto row_factors = [&](int i, float rs[16]) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        rs[r] = a.row_scale[min<int64_t>(m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3), a.M - 1)];
    };
    if (m0 + GBM <= a.M && n0 + GBN <= a.N && extent < (int64_t(1) << 32) && (a.ldy % 2) == 0) {
      const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y, (short)0, (int)(uint32_t)extent, 0x00020000);
      const uint32_t ldyb = (uint32_t)a.ldy * ESZ;
      const uint32_t tile_off = __builtin_amdgcn_readfirstlane((uint32_t)(m0 + wm * 128) * ldyb + (uint32_t)(n0 + wn * 128) * ESZ);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float rs[16];
        row_factors(i, rs);
        if constexpr (EPI == EPI_BF16) {
          const bool odd = (li & 1) != 0;
          const uint32_t voff = (uint32_t)(4 * h) * ldyb + (uint32_t)li * 2 + (odd ? ldyb - 2 : 0u);
          const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int p = 0; p < 8; ++p) {
              typedef float f32x2 __attribute__((ext_vector_type(2)));
              typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
              const f32x2 v = {(acc[i][j][2 * p] * alpha[j]) * rs[2 * p], (acc[i][j][2 * p + 1] * alpha[j]) * rs[2 * p + 1]};
              const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
              const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp((int)pk, (int)pk, 0xB1, 0xF, 0xF, false);
              const uint32_t word = __builtin_amdgcn_perm(nb, pk, sel);
              const uint32_t soff = tile_off + (uint32_t)(i * 32 + 8 * (p >> 1) + 2 * (p & 1)) * ldyb + (uint32_t)(j * 64);
              __builtin_amdgcn_raw_buffer_store_b32(word, yr, voff, soff, 2);
            }
        } else {
          const uint32_t voff = (uint32_t)(4 * h) * ldyb + (uint32_t)li * 4;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t soff = tile_off + (uint32_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldyb + (uint32_t)(j * 128);
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((acc[i][j][r] * alpha[j]) * rs[r]), yr, voff, soff, 2);
            }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float rs[16];
      row_factors(i, rs);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 128 + j * 32 + li;
        const bool n_ok = n < a.N;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (n_ok && m < a.M) store_out_rc<EPI>(a, m, n, acc[i][j][r], alpha[j], rs[r]);
        }
      }
    }
  } else {
    auto scaled = [&](int i, int j, int r) { return acc[i][j][r] * alpha[j]; };
    if (m0 + GBM <= a.M && n0 + GBN <= a.N && extent < (int64_t(1) << 32) && (a.ldy % 2) == 0) {
      const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y, (short)0, (int)(uint32_t)extent, 0x00020000);
      const uint32_t ldyb = (uint32_t)a.ldy * ESZ;
      // wave-uniform (wm, wn are per wave); readfirstlane tells the compiler so
      const uint32_t tile_off = __builtin_amdgcn_readfirstlane((uint32_t)(m0 + wm * 128) * ldyb + (uint32_t)(n0 + wn * 128) * ESZ);
      if constexpr (EPI == EPI_BF16) {
        const bool odd = (li & 1) != 0;
        const uint32_t voff = (uint32_t)(4 * h) * ldyb + (uint32_t)li * 2 + (odd ? ldyb - 2 : 0u);
        const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int p = 0; p < 8; ++p) {
              typedef float f32x2 __attribute__((ext_vector_type(2)));
              typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
              const f32x2 v = {scaled(i, j, 2 * p), scaled(i, j, 2 * p + 1)};
              const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
              const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp((int)pk, (int)pk, 0xB1, 0xF, 0xF, false);
              const uint32_t word = __builtin_amdgcn_perm(nb, pk, sel);
              const uint32_t soff = tile_off + (uint32_t)(i * 32 + 8 * (p >> 1) + 2 * (p & 1)) * ldyb + (uint32_t)(j * 64);
              __builtin_amdgcn_raw_buffer_store_b32(word, yr, voff, soff, 2);
            }
      } else {
        const uint32_t voff = (uint32_t)(4 * h) * ldyb + (uint32_t)li * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t soff = tile_off + (uint32_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldyb + (uint32_t)(j * 128);
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(scaled(i, j, r)), yr, voff, soff, 2);
            }
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 128 + j * 32 + li;
      const bool n_ok = n < a.N;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (n_ok && m < a.M) store_out<EPI>(a, m, n, acc[i][j][r], alpha[j]);
        }
    }
  }
}


}  // namespace

template <int EPI, bool RC>
static hipError_t launch_gemm_epi(const GemmArgs& a, hipStream_t s) {
  // k_gemm_big addresses each packed operand with 32-bit offsets
  const bool offsets32 = a.M * (a.K / 2) < (int64_t(1) << 31) && a.N * (a.K / 2) < (int64_t(1) << 31);
  if (EPI != EPI_GATE && a.K % GBK == 0 && a.K >= 3 * GBK && a.M >= 512 && a.N >= 512 && offsets32) {
    const int64_t big_tiles = ((a.M + GBM - 1) / GBM) * ((a.N + GBN - 1) / GBN);
    if constexpr (EPI != EPI_GATE) {
      hipLaunchKernelGGL((k_gemm_big<EPI, RC>), dim3((unsigned)big_tiles), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  const int64_t tiles = ((a.M + TBM - 1) / TBM) * ((a.N + TBN - 1) / TBN);
  if (a.K % 64 == 0)
    hipLaunchKernelGGL((k_gemm_tiled<true, EPI, RC>), dim3((unsigned)tiles), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm_tiled<false, EPI, RC>), dim3((unsigned)tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t s) {
  if (a.row_scale != nullptr || a.col_scale != nullptr) {
    if (a.row_scale == nullptr || a.col_scale == nullptr || a.gate.n_heads > 0) return hipErrorInvalidValue;
    if (a.y_type == OutType::BF16) return launch_gemm_epi<EPI_BF16, true>(a, s);
    return launch_gemm_epi<EPI_F32, true>(a, s);
  }
  if (a.gate.n_heads > 0) return launch_gemm_epi<EPI_GATE, false>(a, s);
  if (a.y_type == OutType::BF16) return launch_gemm_epi<EPI_BF16, false>(a, s);
  return launch_gemm_epi<EPI_F32, false>(a, s);
}

}  // namespace nvfp4
