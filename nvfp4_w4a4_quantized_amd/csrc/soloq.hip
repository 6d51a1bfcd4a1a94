// Rotated NVFP4 front end (SoloQ-N): each row x is rotated, z = Pi x with
// Pi = (Q_k (x) I_h) blkdiag(H_h D_1, ..., H_h D_k) P, then quantized to NVFP4 with
// global scales computed from the rotated rows themselves, and the scale-only bias
// correction c_bc(z) = ||z||^2 / <q(z), z> is produced per row.
//
// Source: "SoloQ: Calibration-Free Quantization for Diffusion Language Models" page:
// "how it is used" section (the K-RPBH rotation: H_h the normalized Walsh-Hadamard
// matrix, D_i Rademacher signs, P a uniform permutation, Q_k a Haar-random orthogonal
// cross-block mixer), "assumptions and limits" section (x' = Pi x online, W' = W Pi^T
// offline, NVFP4 with scales from the tensor itself, c_bc folded into the per-row
// scales).
//
// The rotated values decide the codes, so they are computed in one fixed fp32 order:
// gather x[perm[i]], apply the sign, the Walsh-Hadamard butterflies stage by stage
// (pair distance 1, 2, 4, ..., h/2; lower <- a + b, upper <- a - b), one multiply by
// fp32(1/sqrt(h)), then per output block r the left-to-right sum
// Q[r][0] y_0 + Q[r][1] y_1 + ... of separately rounded products.  Every step is an
// fp32 add, subtract or multiply rounded once, so any implementation of this order
// gives the same bits.
//
// Layout: one wave = one row at a time (waves loop over rows).  The row of x is staged
// in LDS for the gather.  Lane l holds positions 8l .. 8l+7 of every h = 512 block, so
// the butterflies of distance 1, 2, 4 stay in the lane and those of distance 8 .. 256
// pair lane l with lane l ^ (distance / 8), whose value comes by DPP or a permlane swap
// (no LDS round trip): the lower lane forms v + p, the upper p - v, as fma(+-1, v, p)
// (exact sign, one rounding).  The cross-block mix is in the lane
// (the same positions of every block).  An NVFP4 block (16 consecutive positions) is
// lanes 2b, 2b+1 of one 512-block: its amax is a max over the lane pair.
#include "kernel_common.hpp"

#include <atomic>

namespace nvfp4 {

namespace {

constexpr int RQ_H = 512;                // rotation block size h
constexpr int RQ_WAVES = 4;              // waves (rows in flight) per workgroup

struct RotArgs {
  const void* x;
  int64_t rows, K, ldx;
  const int32_t* perm;
  const int8_t* signs;
  const float* Q;                        // [k][k] row-major
  SegTable seg;
  const float* gvec;                     // QUANT: global scale per segment
  float* gout;                           // AMAX: per-segment atomic max target
  uint8_t* codes;
  uint8_t* scales;
  float* cbc;
  float* z_out;                          // optional [rows][K] fp32
};

template <InType T>
__device__ __forceinline__ float lds_elem(const uint8_t* row, uint32_t idx) {
  if constexpr (T == InType::BF16) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[idx] << 16);
  } else {
    return reinterpret_cast<const float*>(row)[idx];
  }
}

// The value of lane l ^ m (m = 1 .. 32, a constant after unrolling), in VALU: DPP quad
// permutations for m = 1, 2; row rotations by 12 and 4 for m = 4 (l + 4 for lanes with
// bit 2 clear, l - 4 for the others); a rotation by 8 within the 16-lane row for m = 8;
// v_permlane16_swap / v_permlane32_swap of the value with itself for m = 16, 32 (the two
// results hold the lower and the upper row's / half's value).
__device__ __forceinline__ float lane_xor(float v, int m, int lane) {
  const int b = __float_as_int(v);
  switch (m) {
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false));
    case 4: {
      const int up = __builtin_amdgcn_update_dpp(0, b, 0x12C, 0xF, 0xF, false);    // row_ror:12
      const int dn = __builtin_amdgcn_update_dpp(0, b, 0x124, 0xF, 0xF, false);    // row_ror:4
      return __int_as_float((lane & 4) ? dn : up);
    }
    case 8: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, false));   // row_ror:8
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
      return __uint_as_float((lane & 16) ? r[0] : r[1]);
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
      return __uint_as_float((lane & 32) ? r[0] : r[1]);
    }
  }
}

template <InType T, int KB, bool QUANT>
__global__ __launch_bounds__(64 * RQ_WAVES) void k_rotate(RotArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t rq_lds[];
  // AMAX: the workgroup's largest |z| per segment (fp32 bits; non-negative values order
  // as their bits), folded into the global maximum once per workgroup and segment
  __shared__ uint32_t seg_amax[kMaxSeg];
  constexpr int ESZ = (T == InType::BF16) ? 2 : 4;
  constexpr int KD = KB * RQ_H;                                  // row length
  // bf16 rows come into LDS by direct-to-LDS loads one row ahead of their use (two
  // row buffers per wave, no registers held for them); fp32 rows (the offline weight
  // rotation) are staged through registers into one buffer
  constexpr bool DMA = (T == InType::BF16);
  constexpr int NBUF = DMA ? 2 : 1;
  constexpr int NCH = KD * ESZ / 1024;                           // 1 KiB pieces of a row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  uint8_t* const row_base = rq_lds + wave * NBUF * KD * ESZ;
  if constexpr (!QUANT) {
    if ((int)threadIdx.x < a.seg.n) seg_amax[threadIdx.x] = 0u;
    __syncthreads();
  }

  // gather table: position s*512 + 8*lane + j reads element perm[...], sign in bit 15
  uint32_t po[KB * 4];
#pragma unroll
  for (int s = 0; s < KB; ++s)
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const int pos = s * RQ_H + 8 * lane + j;
      const uint32_t i0 = (uint32_t)min(max(a.perm[pos], 0), KD - 1);
      const uint32_t i1 = (uint32_t)min(max(a.perm[pos + 1], 0), KD - 1);
      const uint32_t n0 = a.signs[pos] < 0 ? 0x8000u : 0u;
      const uint32_t n1 = a.signs[pos + 1] < 0 ? 0x8000u : 0u;
      po[s * 4 + j / 2] = (i0 | n0) | ((i1 | n1) << 16);
    }
  const float hs = 0.044194173824159216f;                       // fp32(1 / sqrt(512))

  const int64_t nwaves = (int64_t)gridDim.x * RQ_WAVES;
  // row r -> LDS: NCH loads of 16 bytes per lane (lane l's bytes at piece + 16 l), through
  // a buffer descriptor whose base is the row (no 32-bit limit on the offset into x)
  auto dma_row = [&](int64_t r, uint8_t* buf) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.x) + r * a.ldx * ESZ;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), (short)0, KD * ESZ, 0x00020000);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(buf + 1024 * c), 16,
                                               (uint32_t)(16 * lane), 1024 * c, 0, 0);
  };
  int64_t row = (int64_t)blockIdx.x * RQ_WAVES + wave;
  int cur = 0;
  if constexpr (DMA) {
    if (row < a.rows) dma_row(row, row_base);
  }
  for (; row < a.rows; row += nwaves, cur ^= (NBUF - 1)) {
    uint8_t* const row_lds = row_base + cur * KD * ESZ;
    if constexpr (DMA) {
      // the next row into the other buffer (read two rows ago: that gather has completed),
      // then wait for this row's loads; the stores of the previous row, issued after
      // them, are waited for too (long complete by then)
      if (row + nwaves < a.rows) {
        dma_row(row + nwaves, row_base + (cur ^ 1) * KD * ESZ);
        wait_vmcnt<NCH>();
      } else {
        wait_vmcnt<0>();
      }
    } else {
      // stage the row in LDS (16-byte pieces)
      const uint8_t* src = reinterpret_cast<const uint8_t*>(a.x) + row * a.ldx * ESZ;
      constexpr int NPC = KD * ESZ / 16;
      for (int i = lane; i < NPC; i += 64)
        *reinterpret_cast<u32x4*>(row_lds + 16 * i) = *reinterpret_cast<const u32x4*>(src + 16 * i);
      __builtin_amdgcn_s_waitcnt(0xC07F);                        // lgkmcnt(0): this wave's LDS writes
    }
    __builtin_amdgcn_wave_barrier();

    // gather with signs
    float y[KB][8];
#pragma unroll
    for (int s = 0; s < KB; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t e = (po[s * 4 + j / 2] >> (16 * (j & 1))) & 0xFFFFu;
        const float v = lds_elem<T>(row_lds, e & 0x7FFFu);
        y[s][j] = __uint_as_float(__float_as_uint(v) ^ ((e & 0x8000u) << 16));
      }
    __builtin_amdgcn_wave_barrier();                             // the LDS row may be refilled

    // butterflies of distance 1, 2, 4 (in the lane)
#pragma unroll
    for (int s = 0; s < KB; ++s)
#pragma unroll
      for (int d = 1; d < 8; d *= 2)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((j & d) == 0) {
            const float p = y[s][j], q = y[s][j + d];
            y[s][j] = p + q;
            y[s][j + d] = p - q;
          }
    // distances 8 .. 256: lane l ^ m, m = distance / 8
#pragma unroll
    for (int m = 1; m < 64; m *= 2) {
      const float sg = (lane & m) ? -1.0f : 1.0f;
#pragma unroll
      for (int s = 0; s < KB; ++s) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = lane_xor(y[s][j], m, lane);
          y[s][j] = __builtin_fmaf(sg, y[s][j], p);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < KB; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) y[s][j] = y[s][j] * hs;

    // cross-block mix: z_r = sum_s Q[r][s] y_s, left to right, products rounded first;
    // position by position, in place (y[.][j] is read completely before it is replaced)
    const float* const Qm = a.Q;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float t[KB];
#pragma unroll
      for (int r = 0; r < KB; ++r) {
        t[r] = Qm[r * KB] * y[0][j];
#pragma unroll
        for (int s = 1; s < KB; ++s) t[r] = t[r] + Qm[r * KB + s] * y[s][j];
      }
#pragma unroll
      for (int r = 0; r < KB; ++r) y[r][j] = t[r];
    }
    float (&z)[KB][8] = y;

    int sgi = 0;
    while (sgi + 1 < a.seg.n && row >= a.seg.end[sgi]) ++sgi;
    if constexpr (!QUANT) {
      float am = 0.0f;
#pragma unroll
      for (int r = 0; r < KB; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) am = __builtin_fmaxf(am, __builtin_fabsf(z[r][j]));
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, off));
      if (lane == 0) atomicMax(&seg_amax[sgi], __float_as_uint(am));
    } else {
      const float g = a.gvec[sgi];
      const ScaleConsts sc = scale_consts(g);
      float zz = 0.0f, qz = 0.0f;
      uint8_t* crow = a.codes + row * (a.K >> 1);
      uint8_t* srow = a.scales + row * (a.K >> 4);
#pragma unroll
      for (int r = 0; r < KB; ++r) {
        float am = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) am = __builtin_fmaxf(am, __builtin_fabsf(z[r][j]));
        am = __builtin_fmaxf(am, dpp_swap_adjacent(am));         // the NVFP4 block: lanes 2b, 2b+1
        const uint32_t sb = block_scale_byte(am, sc);
        const uint32_t w = quant8(z[r], sb, g);
        *reinterpret_cast<uint32_t*>(crow + r * (RQ_H / 2) + 4 * lane) = w;
        if ((lane & 1) == 0) srow[r * (RQ_H / 16) + (lane >> 1)] = (uint8_t)sb;
        if (a.z_out) {
          f32x4* zp = reinterpret_cast<f32x4*>(a.z_out + row * a.K + r * RQ_H + 8 * lane);
          zp[0] = f32x4{z[r][0], z[r][1], z[r][2], z[r][3]};
          zp[1] = f32x4{z[r][4], z[r][5], z[r][6], z[r][7]};
        }
        // c_bc parts: ||z||^2 and <e2m1, z> of this block, the latter times s (g at the end)
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const f32x2 e2[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0),
                             __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1),
                             __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2),
                             __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3)};
        float ez = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          ez = __builtin_fmaf(e2[j / 2][0], z[r][j], ez);
          ez = __builtin_fmaf(e2[j / 2][1], z[r][j + 1], ez);
          zz = __builtin_fmaf(z[r][j], z[r][j], zz);
          zz = __builtin_fmaf(z[r][j + 1], z[r][j + 1], zz);
        }
        qz = __builtin_fmaf(e4m3_to_f32(sb), ez, qz);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        zz += __shfl_xor(zz, off);
        qz += __shfl_xor(qz, off);
      }
      qz *= g;
      if (lane == 0) a.cbc[row] = qz > 0.0f ? zz / qz : 1.0f;
    }
  }
  if constexpr (!QUANT) {
    // g = fp32(amax / 2688) is monotone in amax: the largest g is the g of the largest amax
    __syncthreads();
    if ((int)threadIdx.x < a.seg.n && seg_amax[threadIdx.x] != 0u)
      atomicMax(reinterpret_cast<unsigned int*>(a.gout + threadIdx.x),
                __float_as_uint(global_scale_from_amax(__uint_as_float(seg_amax[threadIdx.x]))));
  }
}

// Compute units of the current device, looked up once per device.  The rotation
// kernel holds one wave per SIMD (its registers), so one workgroup per compute unit
// is resident; a grid of that many keeps every wave on its rows for the whole launch
// (8 rows each at 8192 rows), which hides the next row's load behind the current one
// for all but the first row of a wave.
int cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <InType T, int KB>
hipError_t launch_kb(const RotArgs& a, bool quant, hipStream_t s) {
  constexpr int ESZ = (T == InType::BF16) ? 2 : 4;
  const size_t lds = (size_t)RQ_WAVES * (T == InType::BF16 ? 2 : 1) * KB * RQ_H * ESZ;
  const int64_t want = (a.rows + RQ_WAVES - 1) / RQ_WAVES;
  const int64_t cap = cu_count();
  const unsigned grid = (unsigned)(want < cap ? want : cap);
  hipError_t e;
  if (quant) {
    e = lds_limit_once<&k_rotate<T, KB, true>>((int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_rotate<T, KB, true>), dim3(grid), dim3(64 * RQ_WAVES), lds, s, a);
  } else {
    e = lds_limit_once<&k_rotate<T, KB, false>>((int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_rotate<T, KB, false>), dim3(grid), dim3(64 * RQ_WAVES), lds, s, a);
  }
  return hipGetLastError();
}

template <InType T>
hipError_t launch_t(const RotArgs& a, bool quant, hipStream_t s) {
  switch (a.K / RQ_H) {
    case 1: return launch_kb<T, 1>(a, quant, s);
    case 2: return launch_kb<T, 2>(a, quant, s);
    case 4: return launch_kb<T, 4>(a, quant, s);
    case 8: return launch_kb<T, 8>(a, quant, s);
    case 10: return launch_kb<T, 10>(a, quant, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool rotate_shape_ok(int64_t K, int32_t h) {
  if (h != RQ_H || K % RQ_H) return false;
  const int64_t k = K / RQ_H;
  return k == 1 || k == 2 || k == 4 || k == 8 || k == 10;
}

hipError_t launch_rotate_quant(const void* x, InType t, int64_t rows, int64_t K, int64_t ldx, const int32_t* perm,
                               const int8_t* signs, const float* Q, const SegTable& seg, bool dynamic,
                               uint8_t* codes, uint8_t* scales, float* seg_gscale_out, float* cbc, float* z_out,
                               hipStream_t s) {
  RotArgs a{};
  a.x = x;
  a.rows = rows;
  a.K = K;
  a.ldx = ldx;
  a.perm = perm;
  a.signs = signs;
  a.Q = Q;
  a.seg = seg;
  a.gvec = seg_gscale_out;
  a.gout = seg_gscale_out;
  a.codes = codes;
  a.scales = scales;
  a.cbc = cbc;
  a.z_out = z_out;
  hipError_t e;
  if (dynamic) {
    e = launch_fill(seg_gscale_out, seg.n, nullptr, s);          // the atomic max starts from 0
    if (e != hipSuccess) return e;
    e = (t == InType::BF16) ? launch_t<InType::BF16>(a, false, s) : launch_t<InType::F32>(a, false, s);
  } else {
    e = launch_fill(seg_gscale_out, seg.n, &seg, s);             // the calibrated scales
  }
  if (e != hipSuccess) return e;
  return (t == InType::BF16) ? launch_t<InType::BF16>(a, true, s) : launch_t<InType::F32>(a, true, s);
}

}  // namespace nvfp4
