// Device helpers shared by the forward and backward kernels of the fused
// attention library (gfx950).  Included by each kernel source; everything has
// internal linkage.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "fa_mi355x.h"

namespace {

constexpr int kWave = 64;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma_pv(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// f(integral_constant<int, I>) for I = B .. E-1, in order (compile-time loop).
template <int I, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

// Scheduling shape for a run of NM MFMAs fed by RPM LDS reads each: the reads
// of the first LA MFMAs go first, then every MFMA is followed by the reads of
// the MFMA LA places later.  Without it the compiler issues each read right
// before its MFMA and every MFMA waits out the full LDS latency.
template <int NM, int RPM, int LA>
__device__ __forceinline__ void mfma_read_pipeline() {
  static_assert(LA <= NM, "look-ahead longer than the run");
  __builtin_amdgcn_sched_group_barrier(0x100, RPM * LA, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < NM - LA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
}

// Lanes l and l^32 hold the same query.  v_permlane32_swap with both operands
// equal to x leaves each lane holding {x[l], x[l^32]} across its two results,
// so a symmetric combination of the pair reduces over the two lanes.
__device__ __forceinline__ float max_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 h = {(_Float16)lo, (_Float16)hi};  // v_cvt_pk_f16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// Buffer resource over one head's N rows (row r at byte r * row_stride, each
// row_bytes long): loads past the last row return zeros, which is how ragged
// tails are read without bounds branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint8_t* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, nbytes,
                                           0x00020000);
}

// LDS rows are stored with their 16-byte chunks permuted by an XOR swizzle,
// chunk' = chunk ^ f(row), f(row) = 5 * (row / P) mod CPR, where CPR is the
// number of chunks in a row and P = 256 / row_bytes rows share one pass over
// the 64 banks.  f has period 16 in row.  It makes the MFMA operand reads
// conflict-free: 16 consecutive rows read at one logical chunk hit 16
// distinct bank groups, and the 8 rows x 64 bytes of a transposed V read
// spread evenly over the banks.
template <int ROWB>
__device__ __forceinline__ int swz(int row) {
  constexpr int CPR = ROWB / 16;
  constexpr int P = ROWB >= 256 ? 1 : 256 / ROWB;
  return (5 * (row / P)) & (CPR - 1);
}

typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from a buffer straight into LDS: lane t writes
// lds_dst + 16 t (lds_dst must be wave-uniform); past-the-end lanes write 0.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds_dst,
                                                int voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds_dst, 16, voffset, soffset, 0, 0);
}

// Workgroup -> (head, query tile).  Workgroups are dispatched round-robin over
// the device's n_xcd XCDs (workgroup w runs on XCD w % n_xcd), and each XCD
// has its own L2.  When the head count is a multiple of n_xcd, XCD x gets
// heads x, x + n_xcd, ... so all query tiles of a head, which re-read the
// same K and V, share one L2.  Within an XCD, causal work goes longest tiles
// first (the last query tile of each of its heads, then the one before, ...);
// non-causal work goes head by head.
__device__ __forceinline__ void tile_of(int w, int n_heads, int n_tiles, bool causal, int n_xcd,
                                        int& bh, int& qt) {
  int head_slot, rank, heads_here, xcd = 0, stride = 1;
  if (n_xcd > 1 && n_heads % n_xcd == 0) {
    xcd = w % n_xcd;
    w /= n_xcd;
    heads_here = n_heads / n_xcd;
    stride = n_xcd;
  } else {
    heads_here = n_heads;
  }
  if (causal) {
    head_slot = w % heads_here;
    rank = w / heads_here;
    qt = n_tiles - 1 - rank;
  } else {
    head_slot = w / n_tiles;
    qt = w % n_tiles;
  }
  bh = head_slot * stride + xcd;
}

// Compute units and XCDs of the current device, read from the runtime once
// per device and cached; launch shapes, the workgroup -> XCD mapping and the
// key-range split plan depend on them.  If the runtime cannot tell, a whole
// MI355X is assumed (256 CUs in 8 XCDs).  Called only after a call's
// arguments have been validated.
struct Topology {
  int cus;
  int xcds;
};

inline Topology device_topology() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // cus << 8 | xcds; 0: not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return {256, 8};
  }
  if (dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c != 0) return {c >> 8, c & 255};
  }
  int cus = 0, xcds = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0 || cus >= (1 << 20)) {
    (void)hipGetLastError();
    cus = 256;
  }
  if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
      xcds <= 0 || xcds > 255) {
    (void)hipGetLastError();
    xcds = cus == 256 ? 8 : 1;
  }
  if (dev < kMaxDevices) cache[dev].store(cus << 8 | xcds, std::memory_order_relaxed);
  return {cus, xcds};
}

}  // namespace
