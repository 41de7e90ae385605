// gdr_device.h -- device helpers for the gfx950 chunked gated-delta-rule kernels.
//
// Workgroups are 256 threads = 4 wave64.  Chunk GEMMs run on the CDNA4 matrix
// cores: bf16 operands use V_MFMA_F32_16X16X32_BF16, fp32 operands use
// V_MFMA_F32_16X16X4_F32; both accumulate in fp32.  Operand tiles live in LDS.
//
// MFMA lane layouts (wave64, checked on the device):
//   A fragment (16 x KSTEP): lane l holds row l%16, k = 8*(l/16)+j (bf16, j<8)
//                                                  k = l/16         (fp32)
//   B fragment (KSTEP x 16): lane l holds col l%16, same k as A
//   C/D 16 x 16 fp32:        lane l holds rows 4*(l/16)+j (j<4), col l%16
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gdr_kernels.h"

namespace gdr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int CH = 64;      // chunk length (tokens)
constexpr int NTHR = 256;   // threads per workgroup
constexpr int NWAVE = 4;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// The wave index is wave-uniform: read it into a scalar register so that
// branches and addresses derived from it stay scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Orders LDS traffic between the lanes of one wave (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also waits
// for every outstanding global load and store of the wave (vmcnt(0)), which
// would stall on the next chunk's prefetch and on pending output stores; here
// each wave waits for its own LDS operations (lgkmcnt(0)) and then meets the
// others at s_barrier.  Global data that other waves read through LDS is
// always moved there by LDS stores, which this covers.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt = max, expcnt = max, lgkmcnt = 0
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup-wide OR of a per-thread flag through LDS (flags[NW] scratch),
// without the memory fence of __syncthreads_or.
template <int NW>
__device__ __forceinline__ bool lds_any(int pred, int* flags) {
  const bool wave_any = __builtin_amdgcn_ballot_w64(pred != 0) != 0;
  if ((threadIdx.x & 63) == 0) flags[threadIdx.x >> 6] = wave_any ? 1 : 0;
  lds_barrier();
  int any = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) any |= flags[i];
  return any != 0;
}

template <typename T> __device__ __forceinline__ float to_f(T x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f(float x) { return static_cast<T>(x); }

// ------------------------------------------------------- raw buffers --
// Tile loads and stores go through raw buffer descriptors whose record count
// covers exactly the tile's valid rows: the hardware returns zero for loads
// and drops stores outside that range, so partial chunks need no per-row
// branches, and offsets are 32-bit.  Word 3 is the gfx9-family default.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}
// The same descriptor for a base and range that are equal across the wave
// but that the compiler cannot prove uniform: both are taken from the first
// active lane, so the descriptor lives in scalar registers (a descriptor in
// vector registers makes every buffer access a loop over distinct values).
__device__ __forceinline__ rsrc_t make_rsrc_u(const void* base, long bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return make_rsrc((const void*)(uintptr_t)(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane((int)bytes));
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  uint4 u;
  __builtin_memcpy(&u, &v, 16);
  return u;
}
// NT: the non-temporal hint, for data that no later kernel of the call reads
template <bool NT = false>
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, uint4 u) {
  decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)) v;
  __builtin_memcpy(&v, &u, 16);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, NT ? 2 : 0);
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// LDS row pitch (elements) for a row of D elements: +16 bytes keeps 16-byte
// alignment and shifts consecutive rows by four banks.
template <typename T, int D> struct Pitch { static constexpr int value = D + 16 / (int)sizeof(T); };

// ---------------------------------------------------------------- MFMA --
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int KSTEP = 32;
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x4 op(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // Element (i, kk) of a fragment source, i = l%16 (stride RS), kk along K (stride KS).
  template <int RS, int KS>
  __device__ static __forceinline__ frag load(const bf16* p) {
    const int l = lane_id();
    const bf16* q = p + (l & 15) * RS + ((l >> 4) * 8) * KS;
    if constexpr (KS == 1) {
      return *reinterpret_cast<const frag*>(q);
    } else {
      frag f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = q[j * KS];
      return f;
    }
  }
};

template <> struct Mma<float> {
  static constexpr int KSTEP = 4;
  typedef float frag;
  __device__ static __forceinline__ f32x4 op(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  template <int RS, int KS>
  __device__ static __forceinline__ frag load(const float* p) {
    const int l = lane_id();
    return p[(l & 15) * RS + (l >> 4) * KS];
  }
};

// acc[j] += A[16 x KD] * B[KD x 16 (column tile j)], for NT column tiles.
//   A(m, k) = a[m*ARS + k*ACS]          (a points at the tile's (0, 0))
//   B(k, n) = b[k*BRS + (16*j + n)*BCS] (b points at column 0)
// Contraction steps with k0 >= kend are skipped (kend is wave-uniform; the
// skipped part of A must be zero for the result to be exact).
template <typename T, int KD, int NT, int ARS, int ACS, int BRS, int BCS>
__device__ __forceinline__ void mma_row(f32x4 (&acc)[NT], const T* a, const T* b, int kend = KD) {
  constexpr int KS = Mma<T>::KSTEP;
  static_assert(KD % KS == 0, "contraction length must be a multiple of the MFMA K step");
#pragma unroll
  for (int k0 = 0; k0 < KD; k0 += KS) {
    if (k0 < kend) {
      const auto fa = Mma<T>::template load<ARS, ACS>(a + k0 * ACS);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const auto fb = Mma<T>::template load<BCS, BRS>(b + k0 * BRS + 16 * j * BCS);
        acc[j] = Mma<T>::op(fa, fb, acc[j]);
      }
    }
  }
}

// Single 16x16 output tile.
template <typename T, int KD, int ARS, int ACS, int BRS, int BCS>
__device__ __forceinline__ void mma_tile(f32x4& acc, const T* a, const T* b, int kend = KD) {
  f32x4 t[1] = {acc};
  mma_row<T, KD, 1, ARS, ACS, BRS, BCS>(t, a, b, kend);
  acc = t[0];
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Row / column of accumulator element j held by this lane (within a tile).
__device__ __forceinline__ int acc_row(int j) { return 4 * (lane_id() >> 4) + j; }
__device__ __forceinline__ int acc_col() { return lane_id() & 15; }

// ------------------------------------------------------------- staging --
// Global rows -> registers -> LDS.  load() issues every 16-byte global read of
// an R x D tile (rows >= nrows read as zero) before anything is written, so a
// tile's reads overlap; store() writes the rows to LDS (pitch P) and
// store_t() writes the transpose (LDS element (c, r) = scale(r) * tile(r, c)).
template <typename T, int R, int D, int NTH = NTHR>
struct TileRegs {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int VPR = D / VEC;
  static constexpr int NV = (R * VPR + NTH - 1) / NTH;
  static_assert(D % VEC == 0, "row length must be a multiple of 16 bytes");
  uint4 v[NV];
  __device__ __forceinline__ void load(const T* g, long gstride, int nrows) {
    const rsrc_t rr = make_rsrc(g, (long)nrows * gstride * (long)sizeof(T));
    const uint32_t rs = (uint32_t)(gstride * (long)sizeof(T));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = (int)threadIdx.x + i * NTH;
      const int r = idx / VPR, c = idx % VPR;
      if ((R * VPR) % NTH == 0 || idx < R * VPR) v[i] = buf_load16(rr, (uint32_t)r * rs + (uint32_t)c * 16u);
      else v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ int row(int i) const { return ((int)threadIdx.x + i * NTH) / VPR; }
  template <int P>
  __device__ __forceinline__ void store(T* lds) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = (int)threadIdx.x + i * NTH;
      const int r = idx / VPR, c = (idx % VPR) * VEC;
      if (idx < R * VPR) *reinterpret_cast<uint4*>(lds + r * P + c) = v[i];
    }
  }
  template <int PT, typename F>
  __device__ __forceinline__ void store_t(T* lds, F scale) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = (int)threadIdx.x + i * NTH;
      const int r = idx / VPR, c = (idx % VPR) * VEC;
      if (idx < R * VPR) {
        const float s = scale(r);
        const T* e = reinterpret_cast<const T*>(&v[i]);
#pragma unroll
        for (int j = 0; j < VEC; ++j) lds[(c + j) * PT + r] = from_f<T>(to_f(e[j]) * s);
      }
    }
  }
};

// A 64-row tile (rows = tokens) loaded with lane l of every wave on row l and
// the waves splitting the 16-byte column groups.  Its transposed store then
// has consecutive lanes writing consecutive LDS addresses (no bank
// conflicts), and the row store writes one 16-byte group per lane.
template <typename T, int D, int NW = NWAVE>
struct TileCols {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int NCG = D / VEC;
  static constexpr int NV = (NCG + NW - 1) / NW;   // waves beyond NCG groups stay idle
  uint4 v[NV];
  __device__ __forceinline__ void load(const T* g, long gstride, int nrows) {
    const rsrc_t rr = make_rsrc(g, (long)nrows * gstride * (long)sizeof(T));
    const uint32_t off = (uint32_t)lane_id() * (uint32_t)(gstride * (long)sizeof(T));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int cg = wave_id() + NW * i;
      if (NCG % NW == 0 || cg < NCG) v[i] = buf_load16(rr, off + (uint32_t)cg * 16u);
      else v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  template <int P>
  __device__ __forceinline__ void store(T* lds) const {
    const int r = lane_id();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int cg = wave_id() + NW * i;
      if (cg < NCG) *reinterpret_cast<uint4*>(lds + r * P + cg * VEC) = v[i];
    }
  }
  // lds[c * PT + r] = s * tile(r, c), s the scale of this lane's row.
  template <int PT>
  __device__ __forceinline__ void store_t(T* lds, float s) const {
    const int r = lane_id();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int cg = wave_id() + NW * i;
      if (cg < NCG) {
        const T* e = reinterpret_cast<const T*>(&v[i]);
#pragma unroll
        for (int j = 0; j < VEC; ++j) lds[(cg * VEC + j) * PT + r] = from_f<T>(to_f(e[j]) * s);
      }
    }
  }
};

// A 64-row tile loaded like TileCols (lane l of every wave on row l) but with
// wave w holding the contiguous 16-byte column groups [w*NV, (w+1)*NV), i.e.
// elements [w*D/4, (w+1)*D/4) of its row.  store_perm() writes it to LDS with
// the columns permuted: element d of a row goes to column 16*(d % NT) + d / NT
// (NT = D / 16).  The 16 columns of MFMA column tile j then hold the elements
// {NT*c + j : c < 16}, so the accumulators that one lane holds over the NT
// column tiles of a product X * tile are NT consecutive elements of one output
// row, which go back to memory as a single vector store.  Each lane writes
// NT pieces of 4 elements (8 bytes in bf16).
template <typename T, int D>
struct RowSlab {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int NV = D / VEC / NWAVE;
  static constexpr int NT = D / 16;
  static_assert(NV >= 1 && D % (VEC * NWAVE) == 0, "row must split into 16-byte groups over the waves");
  uint4 v[NV];
  __device__ __forceinline__ void load(const T* g, long gstride, int nrows) {
    const rsrc_t rr = make_rsrc(g, (long)nrows * gstride * (long)sizeof(T));
    const uint32_t off = (uint32_t)lane_id() * (uint32_t)(gstride * (long)sizeof(T)) + (uint32_t)(wave_id() * NV * 16);
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = buf_load16(rr, off + (uint32_t)i * 16u);
  }
  template <int P>
  __device__ __forceinline__ void store_perm(T* lds) const {
    T* row = lds + lane_id() * P + 4 * wave_id();
    if constexpr (sizeof(T) == 2) {
      const uint16_t* e = reinterpret_cast<const uint16_t*>(v);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        uint2 pk;
        pk.x = (uint32_t)e[j] | ((uint32_t)e[j + NT] << 16);
        pk.y = (uint32_t)e[j + 2 * NT] | ((uint32_t)e[j + 3 * NT] << 16);
        *reinterpret_cast<uint2*>(row + 16 * j) = pk;
      }
    } else {
      const uint32_t* e = reinterpret_cast<const uint32_t*>(v);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        *reinterpret_cast<uint4*>(row + 16 * j) = make_uint4(e[j], e[j + NT], e[j + 2 * NT], e[j + 3 * NT]);
    }
  }
};

// bf16 MFMA fragment (A or B operand of V_MFMA_F32_16X16X32_BF16) read from a
// row-major LDS matrix M (pitch P elements) whose rows run along the
// contraction: lane l receives M[8*(l/16) + j][l % 16], j < 8, for m pointing
// at the block's (0, 0).  Two DS_READ_B64_TR_B16: within each group of 16
// lanes that instruction gathers a 4 x 16 block, lane s supplying the 8-byte
// piece at row s/4, columns 4*(s%4).., and lane t receiving column t of the
// four rows (lane layout checked on the device).  m must be 8-byte aligned
// and P a multiple of 4.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 tr_frag(const bf16* m, int P) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int l = lane_id(), s = l & 15;
  const bf16* a = m + (8 * (l >> 4) + (s >> 2)) * P + 4 * (s & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + 4 * P));
  bf16x8 f;
  __builtin_memcpy(&f, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&f) + 8, &hi, 8);
  return f;
}

// Four rows r0..r0+3 (r0 may differ between the 16-lane groups) of a
// row-major bf16 LDS matrix at column c0 + l%16: lane l receives
// m[(r0 + i) * P + c0 + l % 16] as element i (one DS_READ_B64_TR_B16).
__device__ __forceinline__ i16x4 tr4(const bf16* m, int P, int r0, int c0) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int s = lane_id() & 15;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(m + (r0 + (s >> 2)) * P + c0 + 4 * (s & 3)));
}
__device__ __forceinline__ bf16x8 cat4(i16x4 lo, i16x4 hi) {
  bf16x8 f;
  __builtin_memcpy(&f, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&f) + 8, &hi, 8);
  return f;
}
// Two 4-element pieces of an LDS row: row[k0 .. k0+3] ++ row[k0+16 .. k0+19].
__device__ __forceinline__ bf16x8 ld_a2(const bf16* row, int k0) {
  const uint2 lo = *reinterpret_cast<const uint2*>(row + k0);
  const uint2 hi = *reinterpret_cast<const uint2*>(row + k0 + 16);
  bf16x8 f;
  __builtin_memcpy(&f, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&f) + 8, &hi, 8);
  return f;
}
// Accumulator tiles X, Y (rows 16b, 16b+16 of a matrix) as the B operand of
// a bf16 MFMA step: lane group q contracts over rows 16b + 4q + j of X
// (j < 4) then the same rows of Y.
__device__ __forceinline__ bf16x8 pack_b(const f32x4& x, const f32x4& y) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = static_cast<bf16>(x[e]);
    f[4 + e] = static_cast<bf16>(y[e]);
  }
  return f;
}
// The second bf16 term of pack_b: the rounding remainders x - hi, y - hi.
__device__ __forceinline__ bf16x8 pack_b_lo(const f32x4& x, const f32x4& y, const bf16x8& hi) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = static_cast<bf16>(x[e] - static_cast<float>(hi[e]));
    f[4 + e] = static_cast<bf16>(y[e] - static_cast<float>(hi[4 + e]));
  }
  return f;
}

__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, uint2 u) {
  decltype(__builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)) v;
  __builtin_memcpy(&v, &u, 8);
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t off, uint32_t u) {
  __builtin_amdgcn_raw_buffer_store_b32(u, r, off, 0, 0);
}

// Row e of this lane's accumulators over NT column tiles (each lane holds
// rows 4*(l/16)+e, column l%16 of every tile) -> NT consecutive elements at
// byte offset off: one 4-, 8- or 16-byte buffer store.
template <typename T, int NT>
__device__ __forceinline__ void store_acc_row(rsrc_t r, uint32_t off, const f32x4 (&acc)[NT], int e) {
  constexpr int BYTES = NT * (int)sizeof(T);
  static_assert(BYTES == 4 || BYTES == 8 || BYTES == 16, "row vector must be 4, 8 or 16 bytes");
  uint32_t w[BYTES / 4];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < NT / 2; ++i) {
      bf16 lo = from_f<bf16>(acc[2 * i][e]), hi = from_f<bf16>(acc[2 * i + 1][e]);
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const float f = acc[i][e];  // bit_cast of a vector element lvalue drops the index
      w[i] = __builtin_bit_cast(uint32_t, f);
    }
  }
  if constexpr (BYTES == 16) buf_store16(r, off, make_uint4(w[0], w[1], w[2], w[3]));
  else if constexpr (BYTES == 8) buf_store8(r, off, make_uint2(w[0], w[1]));
  else buf_store4(r, off, w[0]);
}

// LDS rows [0, nrows) of an R x D tile (pitch P) -> global (row stride gstride),
// 16-byte accesses.
template <typename T, int R, int D, int P, int NTH = NTHR>
__device__ __forceinline__ void store_rows(T* g, long gstride, const T* lds, int nrows) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int VPR = D / VEC;
  const rsrc_t rr = make_rsrc(g, (long)nrows * gstride * (long)sizeof(T));
  const uint32_t rs = (uint32_t)(gstride * (long)sizeof(T));
#pragma unroll
  for (int i = threadIdx.x; i < R * VPR; i += NTH) {
    const int r = i / VPR, c = i % VPR;
    buf_store16(rr, (uint32_t)r * rs + (uint32_t)c * 16u, *reinterpret_cast<const uint4*>(lds + r * P + c * VEC));
  }
}

// Accumulator tile -> LDS, transposed: element (row, col) of the tile goes to
// lds[(col0 + col) * P + row0 + row]; a lane's four rows are contiguous, so
// this is one 8-byte (bf16) or 16-byte (fp32) write.
template <typename T, int P>
__device__ __forceinline__ void acc_store_t(T* lds, int row0, int col0, const f32x4& a, float s = 1.f) {
  T* dst = lds + (col0 + acc_col()) * P + row0 + acc_row(0);
  if constexpr (sizeof(T) == 2) {
    bf16x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = from_f<T>(a[e] * s);
    *reinterpret_cast<bf16x4*>(dst) = pk;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = from_f<T>(a[e] * s);
  }
}

// A'' = A diag(beta) of a chunk (64 x 64 bf16, lower triangular in 16 x 16
// blocks) is stored compactly: row r keeps only its first 32 (r / 16 + 1)
// columns, the blocks on and left of the diagonal, rows one after another
// (5 KB per chunk instead of 8; the zero blocks above the diagonal are not
// stored).  Byte offset of the 16-byte piece pc (< 2 (r / 16 + 1)) of row r,
// and the bytes of the first len rows.
__device__ __forceinline__ uint32_t apack_off(int r, int pc) {
  const int b = r >> 4;
  return (uint32_t)(16 * (16 * b * (b + 1) + (r & 15) * 2 * (b + 1) + pc));
}
__device__ __forceinline__ long apack_bytes(int len) { return (long)apack_off(len, 0); }
// Source offset for a copy of LDS piece pc of row r from the compact rows:
// pieces above the diagonal blocks get an offset past any buffer range, so
// the buffer load returns zeros for them.
__device__ __forceinline__ uint32_t apack_src(int r, int pc) {
  return pc < 2 * ((r >> 4) + 1) ? apack_off(r, pc) : 0x80000000u;
}

// Hardware workgroup id -> logical work index such that each of the 8 XCDs
// (workgroups are dispatched round-robin over them) receives one contiguous
// range of logical indices, run in increasing order: neighbouring work items
// that read the same tiles then share that XCD's L2.  The grid is padded to a
// multiple of 8; indices >= total must exit.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int per = (total + 7) >> 3;
  return (id & 7) * per + (id >> 3);
}

// ---- staged chunk tiles (the fused state kernels) ----
// Staged tiles are unpadded: row r holds NCH 16-byte pieces, piece c stored
// at position c ^ stage_swz(r).  The swizzles were chosen by measured LDS
// throughput on gfx950 for the access patterns of the kernels (8 waves per
// CU, 16-byte MFMA fragment reads of rows 16i + t, 8-byte and transposing
// reads of four-row blocks).  A 16-byte read moves at full rate when the
// pieces that lanes 2m and 2m + 1 read differ only in bit 0, so the row's
// bit 0 goes to the piece's bit 0; for 128-wide rows the other row bits go
// to piece bits 2, 3, 1, which also keeps the transposing reads at the rate
// of the previous layout (row bits 0-2 to piece bits 1-3): fragment reads at
// 228 instead of 128 B per clock and CU.  For 64-wide rows (two rows a
// 256-byte bank line) row bits 1, 2, 3 go to piece bits 0, 2, 1: fragment
// reads at 216 instead of 128, the output pass's 8-byte A'' reads at 172
// instead of 71, transposing reads at 137 instead of 165.
template <int NCH>
__device__ __forceinline__ int stage_swz(int r) {
  if constexpr (NCH == 16) return (r & 1) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 3) | (((r >> 3) & 1) << 1);
  else if constexpr (NCH == 8) return ((r >> 1) & 1) | (((r >> 2) & 1) << 2) | (((r >> 3) & 1) << 1);
  else return (r >> 2) & (NCH - 1);
}

// Global -> LDS copy of 16 (or 4) bytes per lane: BUFFER_LOAD with the LDS
// bit, lane l's bytes landing at lds + 16 l (4 l).  Issued through inline
// assembly on purpose: the compiler's wait-count pass treats every later LDS
// access as possibly aliasing a copy in flight and would wait for all
// copies before it, serialising the copies with the chunk's compute.  The
// kernels that use these wait for the copies themselves (vmcnt(0)) before
// the barrier that publishes the data; nothing else in them uses M0.
typedef int i32x4v __attribute__((ext_vector_type(4)));
// Words of the buffer descriptor that make_rsrc(base, bytes) describes (base
// address, stride 0, byte range, flags), built in wave-uniform registers for
// the inline-assembly copies.  (Taking them from an rsrc_t value goes through
// private memory, which the compiler then places in LDS, one slot per thread.)
__device__ __forceinline__ i32x4v rsrc_words(const void* base, long bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4v v;
  v[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  v[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  v[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  v[3] = kBufWord3;
  return v;
}
// LDS byte address of a pointer into LDS: the low 32 bits of its flat address
// (the shared aperture is 4 GB aligned).  Truncating, rather than casting to
// the LDS address space, keeps the compiler from emitting a null check and a
// 64-bit address per copy (scalar registers it would otherwise spill).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
}
// NT: the non-temporal hint, for tiles read once (no other workgroup of the
// launch reads them), so that they do not displace tiles that others reuse
template <bool NT = false>
__device__ __forceinline__ void lds_copy16(i32x4v rsrc, uint32_t voff, uint32_t lds) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc), "s"(lds) : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds) : "memory");
}
__device__ __forceinline__ void lds_copy4(i32x4v rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds) : "memory");
}

// One wave's share of copying a staged tile from global memory into LDS:
// instruction j fills the 1 KB block w + 8j of the tile; off[j] is this
// lane's byte offset in the source (rows past the descriptor range read 0).
template <int NCP, int NCH, int FNWV, int VEC, bool NT = false, typename T>
__device__ __forceinline__ void lds_copy_tile(T* dst, i32x4v rv, const uint32_t* off, int w) {
#pragma unroll
  for (int j = 0; j < NCP; ++j) {
    const int i = w + FNWV * j;
    if (NCH % FNWV == 0 || i < NCH) lds_copy16<NT>(rv, off[j], lds_addr(dst + 64 * i * VEC));
  }
}

template <int V> using ic = std::integral_constant<int, V>;

constexpr int FNW = 8, FNT = 64 * FNW;   // waves / threads of the fused state kernels

// Sum over the 16 lanes of a DPP row (the lanes sharing lane / 16), on the
// VALU: quad swaps, then the mirrored half-row, then the mirrored row.
template <int C>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), C, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x141>(x);   // row_half_mirror
  x += dpp_f<0x140>(x);   // row_mirror
  return x;
}

// Sixteen row sums at once: on exit lane t of each DPP row holds the sum over
// the row's 16 lanes of x[t].  Four exchange steps with the partners
// t ^ 15 (row mirror), t ^ 7 (half-row mirror), t ^ 2 and t ^ 1 (quad
// swaps); at each step a lane keeps the half of its values whose index bit
// (8, 4, 2, 1) equals its own lane bit and adds the partner's copy of that
// half.  The four masks span all 16 lanes, so every sum has each lane once:
// 45 VALU operations instead of 16 separate reductions (64 DPP adds).
__device__ __forceinline__ float row16_sums16(const float (&x)[16]) {
  const int t = lane_id() & 15;
  float y[8], z[4], u[2];
  {
    const bool b = (t & 8) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = (b ? x[j + 8] : x[j]) + dpp_f<0x140>(b ? x[j] : x[j + 8]);
  }
  {
    const bool b = (t & 4) != 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = (b ? y[j + 4] : y[j]) + dpp_f<0x141>(b ? y[j] : y[j + 4]);
  }
  {
    const bool b = (t & 2) != 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) u[j] = (b ? z[j + 2] : z[j]) + dpp_f<0x4E>(b ? z[j] : z[j + 2]);
  }
  const bool b = (t & 1) != 0;
  return (b ? u[1] : u[0]) + dpp_f<0xB1>(b ? u[0] : u[1]);
}
// Four row sums at once: on exit lane t holds the sum over its DPP row of
// x[t >> 2] (the first two exchange steps of row16_sums16, then plain adds).
__device__ __forceinline__ float row16_sums4(const float (&x)[4]) {
  const int t = lane_id() & 15;
  float y[2];
  {
    const bool b = (t & 8) != 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) y[j] = (b ? x[j + 2] : x[j]) + dpp_f<0x140>(b ? x[j] : x[j + 2]);
  }
  const bool b = (t & 4) != 0;
  float v = (b ? y[1] : y[0]) + dpp_f<0x141>(b ? y[0] : y[1]);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0xB1>(v);
  return v;
}

// 4 x 4 transpose within each quad of lanes: on entry lane 4k + i holds
// x[e] = M[e][i]; on exit x[c] = M[i][c].  Accumulator tiles then give each
// lane four consecutive columns of one row (8-byte bf16 stores).  Two
// exchange steps (partners i ^ 1, then i ^ 2); each output is a select
// between an own value and a partner's, read with a DPP quad permute.
__device__ __forceinline__ f32x4 quad_t(f32x4 x) {
  const int i = lane_id() & 3;
  f32x4 y;
  {
    const bool odd = (i & 1) != 0;
    const float p0 = dpp_f<0xB1>(x[0]), p1 = dpp_f<0xB1>(x[1]), p2 = dpp_f<0xB1>(x[2]), p3 = dpp_f<0xB1>(x[3]);
    y[0] = odd ? p1 : x[0];
    y[1] = odd ? x[1] : p0;
    y[2] = odd ? p3 : x[2];
    y[3] = odd ? x[3] : p2;
  }
  const bool hi = (i & 2) != 0;
  const float p0 = dpp_f<0x4E>(y[0]), p1 = dpp_f<0x4E>(y[1]), p2 = dpp_f<0x4E>(y[2]), p3 = dpp_f<0x4E>(y[3]);
  x[0] = hi ? p2 : y[0];
  x[1] = hi ? p3 : y[1];
  x[2] = hi ? y[2] : p0;
  x[3] = hi ? y[3] : p1;
  return x;
}
__device__ __forceinline__ uint2 pack4_bf16(f32x4 x) {
  bf16x4 b;
#pragma unroll
  for (int c = 0; c < 4; ++c) b[c] = static_cast<bf16>(x[c]);
  uint2 u;
  __builtin_memcpy(&u, &b, 8);
  return u;
}

// CP certificate of one head, called by every thread of the workgroup; cert
// points at the head's first chunk of the sequence.  The per-chunk value is
// the chunk's gate mass, or +inf when a token of the chunk has g > 0 or
// beta |k|^2 outside [0, 2].  With more than one segment, every chunk of the
// sequence must be finite, so that every token transition (forward, and
// transposed in the reverse pass) is a contraction and a warmup error never
// grows after its window; and each warmup window must carry a gate mass of
// at most log_eps: forward windows are the W chunks before a segment start
// that does not reach back to the sequence start; with rev, also the W chunks
// after each segment end that do not reach the sequence end (the reverse pass
// of the backward starts there from zero).
__device__ __forceinline__ bool head_certified(const float* cert, int nseg, int nch, int L, int W,
                                               float log_eps, bool rev) {
  int ok = 1;
  if (nseg > 1)
    for (int cc = (int)threadIdx.x; cc < nch; cc += (int)blockDim.x)
      if (!(cert[cc] <= 0.f)) ok = 0;
  for (int qq = 1 + (int)threadIdx.x; qq < nseg; qq += (int)blockDim.x) {
    const int ws = qq * L - W;
    if (ws > 0) {
      float sum = 0.f;
      for (int cc = ws; cc < qq * L; ++cc) sum += cert[cc];
      if (!(sum <= log_eps)) ok = 0;
    }
    if (rev && qq * L + W < nch) {
      float sum = 0.f;
      for (int cc = qq * L; cc < qq * L + W; ++cc) sum += cert[cc];
      if (!(sum <= log_eps)) ok = 0;
    }
  }
  return !__syncthreads_or(!ok);
}

// Chunk c of the packed batch: its sequence n, first token t0 and length.
__device__ __forceinline__ bool locate_chunk_b(const SeqTables& s, int c, int& n, int& t0, int& len) {
  if (c >= s.NTtot) return false;
  n = s.seq_of_chunk(c);
  t0 = s.cu_at(n) + (c - s.chunk_at(n)) * CH;
  len = min(CH, s.cu_at(n + 1) - t0);
  return len > 0 && t0 >= 0 && (long)t0 + len <= s.Ttot;
}

// Sum over the 16 lanes that share a row of an accumulator tile (lanes with
// equal lane/16); every lane of the group receives the sum.
__device__ __forceinline__ float row_group_sum(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Sum over the four lane groups that share a column (lane % 16).
__device__ __forceinline__ float col_group_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// Four sums over the four lane groups at once: lane 16g + c receives the sum
// over g' of x[g] held by lanes 16g' + c.  Two exchange steps with the
// partners g ^ 1 and g ^ 2; at each a lane keeps the half of its values whose
// index bit matches its own group bit and adds the partner's copy of it.
__device__ __forceinline__ float group_sums4(const float (&x)[4]) {
  const int g = lane_id() >> 4;
  const bool b = (g & 1) != 0;
  float y[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) y[j] = (b ? x[2 * j + 1] : x[2 * j]) + __shfl_xor(b ? x[2 * j] : x[2 * j + 1], 16, 64);
  const bool c = (g & 2) != 0;
  return (c ? y[1] : y[0]) + __shfl_xor(c ? y[0] : y[1], 32, 64);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Inclusive prefix sum across a wave64 (lane i gets x_0 + ... + x_i).
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(x, d, 64);
    if (l >= d) x += y;
  }
  return x;
}

// Shortest warmup of a segment of a certified head: the fewest chunks (at
// most W) whose gate mass already reaches log_eps, taking the window chunks
// first, first + step, ... (step -1: the chunks before a segment start, for
// the forward recurrence; +1: those after a segment end, for the reverse
// pass), of which only `avail` exist.  The state error the warmup leaves is
// bounded by e^(gate mass of the window) times the state's norm whatever the
// window's length, so a shorter window that meets the threshold keeps the
// certificate's bound.  Returns W when no shorter window does (the head
// certificate holds for W, or the window reaches the sequence edge and runs
// exactly).  Called by every lane of a wave, uniform arguments; x0 is this
// lane's value of the first 64 window chunks, loaded ahead by warmup_first()
// so that its latency overlaps the head certificate's loads.
__device__ __forceinline__ float warmup_first(const float* cert, int first, int step, int avail, int W) {
  const int l = lane_id();
  return l < min(W, avail) ? cert[first + step * l] : 0.f;
}
__device__ __forceinline__ int short_warmup(const float* cert, int first, int step, int avail, int W,
                                            float log_eps, float x0) {
  const int l = lane_id();
  const int n = min(W, avail);
  float carry = 0.f;
  for (int b = 0; b < n; b += 64) {
    const int i = b + l;
    const float x = wave_inclusive_scan(b == 0 ? x0 : (i < n ? cert[first + step * i] : 0.f)) + carry;
    const unsigned long long hit = __ballot(i < n && x <= log_eps);
    if (hit) return b + __ffsll((long long)hit);   // lowest hitting lane, 1-based
    carry = __shfl(x, 63, 64);
  }
  return W;
}

}  // namespace gdr
