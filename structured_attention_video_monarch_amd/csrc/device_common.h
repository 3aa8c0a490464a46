// Device helpers shared by the MonarchAttention kernels (gfx950, wave64).
//
// MFMA operand convention used throughout.  For a 16x16 output tile and a
// 32-wide contraction step, lane l (G = l/16) supplies row (A) or column (B)
// index l%16 and eight contraction "slots" 8G..8G+7, stored as one fragment
// of eight elements.  bf16 fragments feed one v_mfma_f32_16x16x32_bf16; f32
// fragments feed eight v_mfma_f32_16x16x4_f32, call j taking slot j of every
// lane group.  Either way A slot (G,j) meets B slot (G,j), so any fixed map
// from slots to contraction indices works as long as both operands use it.
// The output tile gives lane l the rows 4G+i (i = 0..3) of column l%16.
//
// Slot permutation: when an output tile feeds the next product as an
// operand (the softmax weights), the first product loads its A rows in the
// order perm(ct, m) = 8*(m/4) + 4*ct + m%4 for the two 16-row halves ct of a
// 32-row block.  Lane group G then holds rows 8G..8G+7 of the block, which
// is exactly the slot map "slot j <-> index 8G+j" of the next product, and
// the other operand of that product reads eight consecutive elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace monarch {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bf16 storage

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

template <typename T> struct Elem;

template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;  // elements per 16-byte access
  static constexpr int kPad = 8;  // LDS row padding (elements)
  using frag = bf16x8;
  __device__ static inline frag zero() { return frag{}; }
  __device__ static inline frag load(const bf16_t* p) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(p));
  }
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline bf16_t from_f32(float x) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(x));
  }
  __device__ static inline float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
  }
  // eight floats -> fragment (round to nearest even)
  __device__ static inline frag pack(const float* v) {
    frag r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(v[j]);
    return r;
  }
  // eight floats (already in output order) -> one 16-byte store
  __device__ static inline void store8(bf16_t* p, const float* v) {
    frag r = pack(v);
    *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, r);
  }
  __device__ static inline void store4(bf16_t* p, const float* v) {
    uint2 u;
    u.x = static_cast<uint32_t>(from_f32(v[0])) | (static_cast<uint32_t>(from_f32(v[1])) << 16);
    u.y = static_cast<uint32_t>(from_f32(v[2])) | (static_cast<uint32_t>(from_f32(v[3])) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
  // the value a fragment slot holds, as float (for sums of rounded weights)
  __device__ static inline float slot(const frag& f, int j) { return static_cast<float>(f[j]); }
  // Fragment whose contraction index runs down the rows of a row-major LDS
  // tile: lane (G, i) gets tile[k0 + 8G + j][cbase + cstride*(i/4) + i%4],
  // j = 0..7.  Two ds_read_b64_tr_b16: within each 16-lane block, output lane
  // i, element j is element i%4 of the 8 bytes addressed by lane 4j + i/4.
  __device__ static inline frag load_tr(const bf16_t* tile, int pitch, int k0, int cbase,
                                        int cstride) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const int l = threadIdx.x & 63;
    const int i = l & 15, G = l >> 4;
    const bf16_t* p = tile + (k0 + 8 * G + (i >> 2)) * pitch + cbase + cstride * (i & 3);
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * pitch));
    const v8i16 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(frag, r);
  }
};

template <> struct Elem<float> {
  static constexpr int kVec = 4;
  static constexpr int kPad = 4;
  struct frag { f32x4 lo, hi; };
  __device__ static inline frag zero() { return frag{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }
  __device__ static inline frag load(const float* p) {
    frag r;
    r.lo = *reinterpret_cast<const f32x4*>(p);
    r.hi = *reinterpret_cast<const f32x4*>(p + 4);
    return r;
  }
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], c, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], c, 0, 0, 0);
    return c;
  }
  __device__ static inline float from_f32(float x) { return x; }
  __device__ static inline float to_f32(float x) { return x; }
  __device__ static inline frag pack(const float* v) {
    frag r;
#pragma unroll
    for (int j = 0; j < 4; ++j) { r.lo[j] = v[j]; r.hi[j] = v[4 + j]; }
    return r;
  }
  __device__ static inline void store8(float* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
  __device__ static inline void store4(float* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
  __device__ static inline float slot(const frag& f, int j) { return j < 4 ? f.lo[j] : f.hi[j - 4]; }
  // Same contract as the bf16 version, with plain LDS reads.
  __device__ static inline frag load_tr(const float* tile, int pitch, int k0, int cbase,
                                        int cstride) {
    const int l = threadIdx.x & 63;
    const int i = l & 15, G = l >> 4;
    const float* p = tile + (k0 + 8 * G) * pitch + cbase + cstride * (i >> 2) + (i & 3);
    frag r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.lo[j] = p[j * pitch];
      r.hi[j] = p[(4 + j) * pitch];
    }
    return r;
  }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }

// Row of a 32-row block that row slot m of half ct loads (see header).
__device__ inline int perm_row(int ct, int m) { return 8 * (m >> 2) + 4 * ct + (m & 3); }

// Bounds of tile g of the a1 index: floor(g*b1/t).
__device__ inline int tile_lo(int g, int b1, int t) {
  return static_cast<int>((static_cast<long long>(g) * b1) / t);
}

// Spread consecutive logical work items over one XCD: the hardware hands
// workgroup i to XCD i % 8, so items that share inputs through L2 get
// consecutive logical ids on the same XCD.
__device__ inline int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int xcd = bid % kXcd, idx = bid / kXcd;
  const int per = nblocks / kXcd, rem = nblocks % kXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// Register-staged copy of a ROWS x DK tile (row stride `rstride` elements in
// global memory) into an LDS tile of pitch `pitch`.  load() issues the global
// reads; store() writes them to LDS, so a caller can compute on one LDS
// buffer while the next tile is in flight.  Rows >= nvalid and columns >= D
// (up to DK) are zero.
template <typename T, int D, int DK, int ROWS, int NT>
struct TileLoader {
  static constexpr int V = Elem<T>::kVec;
  static constexpr int VPR = DK / V;
  static constexpr int TOTAL = ROWS * VPR;
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  uint4 buf[PER];
  __device__ inline void load(const T* g, long long rstride, int nvalid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = threadIdx.x + u * NT;
      const int r = idx / VPR, c = (idx % VPR) * V;
      buf[u] = uint4{0u, 0u, 0u, 0u};
      if ((TOTAL % NT == 0 || idx < TOTAL) && r < nvalid && c < D)
        buf[u] = *reinterpret_cast<const uint4*>(g + r * rstride + c);
    }
  }
  __device__ inline void store(T* lds, int pitch) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = threadIdx.x + u * NT;
      if (TOTAL % NT != 0 && idx >= TOTAL) break;
      const int r = idx / VPR, c = (idx % VPR) * V;
      *reinterpret_cast<uint4*>(lds + r * pitch + c) = buf[u];
    }
  }
};

}  // namespace monarch
