// MXFP4 variant on gfx950's native block-scaled FP4 MFMA: E2M1 elements with one
// E8M0 (power-of-two) scale per 32 elements and no global scale.  This is the format
// the pages name as the next one to generalize to ("Why Gated DeltaNet Survives
// 4-Bit Quantization" review page, future work / the paper's section 9); the format
// itself follows the public OCP Microscaling definition: shared exponent
// floor(log2(block amax)) - 2, elements rounded to nearest even onto E2M1 and
// saturated at 6.
//
// Unlike NVFP4 (an E4M3 scale per 16 elements, whose products with E2M1 need up to
// 6 significant bits), this format is exactly what v_mfma_scale_f32_32x32x64_f8f6f4
// consumes: the packed codes go from LDS straight into the MFMA with their E8M0
// scales, no decode.
#include "kernel_common.hpp"

namespace nvfp4 {

namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------------
// Quantizer: one lane = one 32-element block (bf16: four 16-byte loads, fp32: eight);
// consecutive lanes take consecutive blocks of a row.
// ---------------------------------------------------------------------------------
template <InType T>
__global__ __launch_bounds__(256) void k_mx_quant(const void* x, int64_t ldx, int64_t K, uint32_t nblk,
                                                  uint32_t bpr, uint8_t* codes, uint8_t* scales) {
  for (uint32_t q = blockIdx.x * blockDim.x + threadIdx.x; q < nblk; q += gridDim.x * blockDim.x) {
    const uint32_t row = q / bpr, cb = q - row * bpr;
    float v[32];
    if constexpr (T == InType::BF16) {
      const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + (int64_t)row * ldx + 32 * cb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 w = __builtin_nontemporal_load(p + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[8 * i + 2 * e] = __uint_as_float(w[e] << 16);
          v[8 * i + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
      }
    } else {
      const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x) + (int64_t)row * ldx + 32 * cb);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4 w = __builtin_nontemporal_load(p + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * i + e] = w[e];
      }
    }
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
    // floor(log2 amax) from the bits (exact; subnormal amax by its leading mantissa bit)
    const uint32_t ab = __float_as_uint(am);
    const int ef = (int)(ab >> 23);
    const int fl = ef != 0 ? ef - 127 : (31 - __builtin_clz(ab | 1u)) - 149;
    const int shared = am > 0.0f ? min(127, max(-127, fl - 2)) : -127;
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = __builtin_ldexpf(v[8 * d + e], -shared);   // exact (or tiny: code 0)
      w[d] = cvt8_fp4(y);
    }
    *reinterpret_cast<u32x4*>(codes + (int64_t)row * (K >> 1) + 16 * cb) = u32x4{w[0], w[1], w[2], w[3]};
    scales[(int64_t)row * (K >> 5) + cb] = (uint8_t)(shared + 127);
  }
}

// ---------------------------------------------------------------------------------
// GEMM: 256 x 256 output tile per workgroup, BK = 64 (two MX blocks), 4 waves of
// 128 x 128 (4 x 4 MFMA 32x32x64 with FP4 operands, fp32 accumulators in AGPRs).
// A lane (h, li) feeds row li of a 32-row block with its 16 bytes of codes for
// elements 32 h .. 32 h + 31 of the K step (= MX block h) and that block's E8M0
// scale.  Packed tiles go HBM -> LDS by direct-to-LDS loads in slots of four K steps
// (a row's 128 bytes of codes = one cache line per load, which is what bounds the
// feed: loads of 32 bytes per row per K step reached only ~4 TB/s of L2->LDS traffic),
// two slots, the next slot loaded while the current one is consumed; operand registers
// are double-buffered and the LDS reads of the next step run under the second half of
// a K step's MFMAs.  Rows past M or N are
// clamped (never stored).  Requires K % 128 == 0 (an even number of K steps).
// ---------------------------------------------------------------------------------
constexpr int XBM = 256, XBN = 256, XBK = 64;
// LDS ring: 2 slots of 4 K steps (256 elements) each.  Slot layout: codes [row][128 B]
// (one whole cache line of the row, 16-byte chunk c stored at chunk c ^ (row & 7), so
// that the per-lane 16-byte reads of 8 consecutive rows hit distinct banks), then the
// row's 8 scale bytes as two dword planes [dword][row][4 B] (direct-to-LDS loads give
// every lane a 4-byte slot).
constexpr int XSS = 4;                                  // K steps per slot
constexpr int XS_A = 0, XS_W = 32768, XS_SA = 65536, XS_SW = 67584, XS_BYTES = 69632;

struct MxArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  int64_t M, N, K;
  void* y;
  int64_t ldy;
};

__device__ __forceinline__ void mx_tile_of(int64_t M, int64_t N, int64_t pid, int64_t* bm, int64_t* bn) {
  // as for the NVFP4 prefill kernel: XCD x (= pid % 8) takes a contiguous range of
  // logical tiles, ordered in groups of 4 row tiles sweeping the column tiles
  const int64_t tiles_m = (M + XBM - 1) / XBM;
  const int64_t tiles_n = (N + XBN - 1) / XBN;
  const int64_t num = tiles_m * tiles_n;
  const int64_t logical = (num % 8 == 0) ? (pid % 8) * (num / 8) + pid / 8 : pid;
  const int64_t group = 4;
  const int64_t per_group = group * tiles_n;
  const int64_t first_m = (logical / per_group) * group;
  const int64_t gsize = (tiles_m - first_m) < group ? (tiles_m - first_m) : group;
  *bm = first_m + (logical % per_group) % gsize;
  *bn = (logical % per_group) / gsize;
}

__device__ __forceinline__ void mx_load_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int size, uint32_t voff, int soff) {
  if (size == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

struct MxRegs {
  u32x4 a[4], b[4];         // 32 FP4 codes per lane (the MFMA reads 4 of its 8 operand registers)
  int32_t sa[4], sb[4];     // E8M0 scale bytes
};

__device__ __forceinline__ i32x8 fp4_operand(u32x4 c) {
  return i32x8{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
}

template <bool BF16OUT>
__global__ __launch_bounds__(256, 1) void k_mx_gemm(MxArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * XS_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, li = lane & 31;
  int64_t bm, bn;
  mx_tile_of(a.M, a.N, blockIdx.x, &bm, &bn);
  const int64_t m0 = bm * XBM, n0 = bn * XBN;
  const int64_t K = a.K, kh = K >> 1, kbs = K >> 5;

  // load roles per slot: 64 rows of A and of W codes per wave, 8 rows per instruction
  // (lane l: row 8 q + l / 8 of the wave's 64, physical chunk l % 8 = logical chunk
  // (l % 8) ^ (row & 7): each row's 128 bytes come from one cache line), and the
  // wave's 64 rows of A and of W scales (two dwords per row).  Rows past M or N are
  // clamped (in bounds; never stored); bytes past a row's end (last, partial slot)
  // are never read by the MFMAs, and past the buffer the descriptor returns zero.
  const int lrow = lane >> 3, lchunk = lane & 7;
  uint32_t oa_c[8], ow_c[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = 64 * wave + 8 * q + lrow;
    const int c = lchunk ^ (row & 7);
    oa_c[q] = (uint32_t)(min<int64_t>(m0 + row, a.M - 1) * kh + 16 * c);
    ow_c[q] = (uint32_t)(min<int64_t>(n0 + row, a.N - 1) * kh + 16 * c);
  }
  const uint32_t lo_c = (uint32_t)(64 * wave * 128);
  const uint32_t oa_s = (uint32_t)(min<int64_t>(m0 + 64 * wave + lane, a.M - 1) * kbs);
  const uint32_t ow_s = (uint32_t)(min<int64_t>(n0 + 64 * wave + lane, a.N - 1) * kbs);
  const uint32_t lo_s = (uint32_t)(64 * wave * 4);
  const __amdgpu_buffer_rsrc_t ra_c = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.a_codes), (short)0,
                                                                        (int)(a.M * kh), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw_c = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.w_codes), (short)0,
                                                                        (int)(a.N * kh), 0x00020000);
  const __amdgpu_buffer_rsrc_t ra_s = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.a_scales), (short)0,
                                                                        (int)(a.M * kbs), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw_s = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.w_scales), (short)0,
                                                                        (int)(a.N * kbs), 0x00020000);
  // slot sl <- K steps 4 s .. 4 s + 3 (elements k0 = 256 s ..)
  auto issue = [&](int sl, int64_t k0) {
    uint8_t* base = smem + sl * XS_BYTES;
    const int kc = (int)(k0 >> 1), ks = (int)(k0 >> 5);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mx_load_lds(ra_c, base + XS_A + lo_c + q * 1024, 16, oa_c[q], kc);
      mx_load_lds(rw_c, base + XS_W + lo_c + q * 1024, 16, ow_c[q], kc);
    }
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      mx_load_lds(ra_s, base + XS_SA + d * 1024 + lo_s, 4, oa_s, ks + 4 * d);
      mx_load_lds(rw_s, base + XS_SW + d * 1024 + lo_s, 4, ow_s, ks + 4 * d);
    }
  };

  // operand reads: row r = w * 128 + 32 i + li, K step sub of the slot: logical chunk
  // 2 sub + h at physical chunk (2 sub + h) ^ (li & 7); scale byte 2 (sub & 1) + h of
  // dword plane sub >> 1
  const uint32_t la_c = (uint32_t)(XS_A + (wm * 128 + li) * 128);
  const uint32_t lw_c = (uint32_t)(XS_W + (wn * 128 + li) * 128);
  const uint32_t la_s = (uint32_t)(XS_SA + (wm * 128 + li) * 4 + h);
  const uint32_t lw_s = (uint32_t)(XS_SW + (wn * 128 + li) * 4 + h);
  const int l7 = li & 7;
  auto lread = [&](int64_t kt, MxRegs& r) {
    const int sub = (int)(kt & 3);
    const uint8_t* base = smem + (int)((kt >> 2) & 1) * XS_BYTES;
    const uint32_t coff = (uint32_t)(16 * ((2 * sub + h) ^ l7));
    const uint8_t* sbase = base + (sub >> 1) * 1024 + 2 * (sub & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.a[i] = *reinterpret_cast<const u32x4*>(base + la_c + coff + i * 4096);
      r.sa[i] = sbase[la_s + i * 128];
      r.b[i] = *reinterpret_cast<const u32x4*>(base + lw_c + coff + i * 4096);
      r.sb[i] = sbase[lw_s + i * 128];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  auto mfma_rows = [&](const MxRegs& r, int i0) {
#pragma unroll
    for (int i = i0; i < i0 + 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(r.a[i]), fp4_operand(r.b[j]),
                                                                     acc[i][j], 4, 4, 0, r.sa[i], 0, r.sb[j]);
  };

  MxRegs R0, R1;
  const int64_t nk = K / XBK;           // even (K % 128 == 0)
  const int64_t nslot = (nk + XSS - 1) / XSS;
  // K step kt with operands in cur; reads step kt+1 into nxt.  At the first step of a
  // slot the loads of the next slot go into the other slot, whose last reads (step
  // kt-1, read during step kt-2) ended before the barrier of step kt-1.  At the last
  // step of a slot every wave waits for its loads of the next slot, then the barrier
  // publishes them; inside a slot no barrier is needed.
  auto kstep = [&](int64_t kt, MxRegs& cur, MxRegs& nxt, bool next) {
    const int64_t sl = kt >> 2;
    if ((kt & 3) == 0 && sl + 1 < nslot) issue((int)((sl + 1) & 1), (sl + 1) * XSS * XBK);
    mfma_rows(cur, 0);
    if (next) {
      if (((kt + 1) & 3) == 0) {
        wait_vmcnt<0>();
        wg_barrier();
      }
      lread(kt + 1, nxt);
    }
    mfma_rows(cur, 2);
  };

  issue(0, 0);
  wait_vmcnt<0>();
  wg_barrier();
  lread(0, R0);
  for (int64_t kt = 0; kt < nk; kt += 2) {
    kstep(kt, R0, R1, true);
    kstep(kt + 1, R1, R0, kt + 2 < nk);
  }
  wait_vmcnt<0>();                      // no direct-to-LDS write may outlive the workgroup

  // Epilogue, one path for every tile.  D of block (i, j): lane (h, li) holds column li,
  // rows 8 (r >> 2) + 4 h + (r & 3).  Stores go through a buffer descriptor of y whose
  // size is y's byte extent: a per-lane VGPR offset fixed for the whole epilogue plus a
  // wave-uniform SGPR offset.  Rows past M lie at or beyond the extent, so the hardware
  // drops their stores; columns past N are masked per lane.  The host guarantees that
  // no offset wraps 32 bits ((M + 264) * ldy * size < 2^32), an even ldy, and for bf16
  // output an even N (pairs of adjacent columns are stored as one 32-bit word, built
  // across neighbouring lanes with DPP, as in the NVFP4 prefill kernel).  The stores
  // are non-temporal (cache policy nt), which keeps the output out of the caches the
  // operand tiles are re-read through: 0.517 -> 0.475 ms at 8192 x 16384 x 5120.
  constexpr int ESZ = BF16OUT ? 2 : 4;
  const int64_t extent = ((a.M - 1) * a.ldy + a.N) * ESZ;
  const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y, (short)0, (int)(uint32_t)extent, 0x00020000);
  const uint32_t ldyb = (uint32_t)a.ldy * ESZ;
  const uint32_t tile_off = __builtin_amdgcn_readfirstlane((uint32_t)(m0 + wm * 128) * ldyb + (uint32_t)(n0 + wn * 128) * ESZ);
  const int64_t ncol = n0 + wn * 128 + (BF16OUT ? (li | 1) : li);   // last column this lane writes, block j = 0
  if constexpr (BF16OUT) {
    const bool odd = (li & 1) != 0;
    const uint32_t voff = (uint32_t)(4 * h) * ldyb + (uint32_t)li * 2 + (odd ? ldyb - 2 : 0u);
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool col_ok = ncol + 32 * j < a.N;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          typedef float f32x2 __attribute__((ext_vector_type(2)));
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          const f32x2 v = {acc[i][j][2 * p], acc[i][j][2 * p + 1]};
          const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
          const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp((int)pk, (int)pk, 0xB1, 0xF, 0xF, false);
          const uint32_t word = __builtin_amdgcn_perm(nb, pk, sel);
          const uint32_t soff = tile_off + (uint32_t)(i * 32 + 8 * (p >> 1) + 2 * (p & 1)) * ldyb + (uint32_t)(j * 64);
          if (col_ok) __builtin_amdgcn_raw_buffer_store_b32(word, yr, voff, soff, 2);
        }
    }
  } else {
    const uint32_t voff = (uint32_t)(4 * h) * ldyb + (uint32_t)li * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool col_ok = ncol + 32 * j < a.N;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t soff = tile_off + (uint32_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldyb + (uint32_t)(j * 128);
          if (col_ok) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), yr, voff, soff, 2);
        }
    }
  }
}

}  // namespace

hipError_t launch_mx_quant(const void* x, InType t, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                           uint8_t* scales, hipStream_t s) {
  const int64_t nblk = M * (K / 32);
  const int64_t want = (nblk + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  if (t == InType::BF16)
    hipLaunchKernelGGL(k_mx_quant<InType::BF16>, dim3(grid), dim3(256), 0, s, x, ldx, K, (uint32_t)nblk,
                       (uint32_t)(K / 32), codes, scales);
  else
    hipLaunchKernelGGL(k_mx_quant<InType::F32>, dim3(grid), dim3(256), 0, s, x, ldx, K, (uint32_t)nblk,
                       (uint32_t)(K / 32), codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                          const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y, bool bf16_out,
                          int64_t ldy, hipStream_t s) {
  MxArgs a{a_codes, a_scales, w_codes, w_scales, M, N, K, y, ldy};
  const unsigned tiles = (unsigned)(((M + XBM - 1) / XBM) * ((N + XBN - 1) / XBN));
  if (bf16_out)
    hipLaunchKernelGGL(k_mx_gemm<true>, dim3(tiles), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_mx_gemm<false>, dim3(tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace nvfp4
