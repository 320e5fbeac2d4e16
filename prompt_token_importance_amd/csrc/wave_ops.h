// Wave-level building blocks shared by the selection kernels (64-lane waves).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

// Inclusive scan over the 64 lanes of a wave through DPP row shifts (within
// rows of 16 lanes) and the two row broadcasts; lanes that a shift or a row
// mask leaves out read the identity `id`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t id, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROWS, 0xF, false);
}

struct OpAdd {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct OpMin {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct OpMax {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};
// float ops on the bit patterns the DPP moves carry
struct OpAddF {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }
};
struct OpMaxF {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }
};

template <class Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t id) {
  Op op;
  v = op(v, dpp_mov<0x111, 0xF>(id, v));   // row_shr:1
  v = op(v, dpp_mov<0x112, 0xF>(id, v));   // row_shr:2
  v = op(v, dpp_mov<0x114, 0xF>(id, v));   // row_shr:4
  v = op(v, dpp_mov<0x118, 0xF>(id, v));   // row_shr:8
  v = op(v, dpp_mov<0x142, 0xA>(id, v));   // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_mov<0x143, 0xC>(id, v));   // row_bcast:31 into rows 2 and 3
  return v;
}

}  // namespace kvs
