// bst_instances.hpp -- the table of compiled kernel instances.  Each
// inst_*.hip translation unit instantiates the kernels of one operand type
// and exports its slice of the table; bst.hip picks an entry per call.
#pragma once

#include <hip/hip_runtime.h>

#include "bst_device.hpp"
#include "bst_kernel_dma.hpp"

namespace bst {

using LaunchFn = hipError_t (*)(dim3, dim3, hipStream_t, const GemmArgs&);

struct Instance {
  int ab;  // AbKind
  int bm, bn;
  int form;    // Form: plain / batched, grouped slice-M, grouped slice-K
  bool dma;    // LDS-DMA family (else register-staged)
  int stages;  // pipeline stages of the LDS-DMA family
  const void* fn;
  LaunchFn launch;
  int threads;
  int bk;
  bool add = false;  // matmul-add epilogue (C = A.B + X)
  int wgs = 1;       // resident workgroups per CU it is built for (2: gemm_dma_kernel_pair)
};

struct InstanceList {
  const Instance* begin;
  int count;
};

template <int AB, int BM, int BN, int WM, int WN, int GR>
hipError_t launch_reg(dim3 grid, dim3 block, hipStream_t st, const GemmArgs& a) {
  hipLaunchKernelGGL((gemm_kernel<AB, BM, BN, WM, WN, GR>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int AB, int BM, int BN, int WM, int WN, int S, int GR, bool ADD = false>
hipError_t launch_dma(dim3 grid, dim3 block, hipStream_t st, const GemmArgs& a) {
  hipLaunchKernelGGL((gemm_dma_kernel<AB, BM, BN, WM, WN, S, GR, ADD>), grid, block, 0, st, a);
  return hipGetLastError();
}

#define BST_REG(AB, BM, BN, WM, WN, GR)                                                   \
  Instance {                                                                              \
    AB, BM, BN, GR, false, 1,                                                             \
        reinterpret_cast<const void*>(&gemm_kernel<AB, BM, BN, WM, WN, GR>),              \
        &launch_reg<AB, BM, BN, WM, WN, GR>, 64 * WM * WN, Traits<AB>::BK                 \
  }
#define BST_DMA(AB, BM, BN, WM, WN, S, GR)                                                \
  Instance {                                                                              \
    AB, BM, BN, GR, true, S,                                                              \
        reinterpret_cast<const void*>(&gemm_dma_kernel<AB, BM, BN, WM, WN, S, GR>),       \
        &launch_dma<AB, BM, BN, WM, WN, S, GR>, 64 * WM * WN, Traits<AB>::BK              \
  }

template <int AB, int BM, int BN, int WM, int WN, int S, int GR>
hipError_t launch_dma_pair(dim3 grid, dim3 block, hipStream_t st, const GemmArgs& a) {
  hipLaunchKernelGGL((gemm_dma_kernel_pair<AB, BM, BN, WM, WN, S, GR>), grid, block, 0, st, a);
  return hipGetLastError();
}

// An LDS-DMA instance built for two resident workgroups per CU.
#define BST_DMA_PAIR(AB, BM, BN, WM, WN, S, GR)                                           \
  Instance {                                                                              \
    AB, BM, BN, GR, true, S,                                                              \
        reinterpret_cast<const void*>(&gemm_dma_kernel_pair<AB, BM, BN, WM, WN, S, GR>),  \
        &launch_dma_pair<AB, BM, BN, WM, WN, S, GR>, 64 * WM * WN, Traits<AB>::BK, false, 2 \
  }

// A matmul-add instance of the LDS-DMA family (plain GEMM only).
#define BST_DMA_ADD(AB, BM, BN, WM, WN, S)                                                \
  Instance {                                                                              \
    AB, BM, BN, FORM_DENSE, true, S,                                                      \
        reinterpret_cast<const void*>(&gemm_dma_kernel<AB, BM, BN, WM, WN, S, FORM_DENSE, true>), \
        &launch_dma<AB, BM, BN, WM, WN, S, FORM_DENSE, true>, 64 * WM * WN, Traits<AB>::BK, true \
  }

InstanceList instances_f16();
InstanceList instances_bf16();
InstanceList instances_i8();
InstanceList instances_fp8();
InstanceList instances_mxfp8();
InstanceList instances_slicek();

}  // namespace bst
