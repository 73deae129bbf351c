// inst_slicek.hip -- compiled kernel instances for grouped slice-K problems
// (int8 with or without dequant, fp16, bf16).
#include "bst_instances.hpp"

namespace bst {

static const Instance kList[] = {
    BST_REG(AB_I8, 64, 64, 2, 2, FORM_SLICE_K),    BST_REG(AB_I8, 128, 128, 2, 2, FORM_SLICE_K),
    BST_REG(AB_I8, 256, 256, 4, 2, FORM_SLICE_K),
    BST_DMA(AB_I8, 64, 64, 2, 2, 4, FORM_SLICE_K),   BST_DMA(AB_I8, 128, 128, 2, 2, 4, FORM_SLICE_K),
    BST_DMA(AB_I8, 256, 128, 2, 2, 3, FORM_SLICE_K), BST_DMA(AB_I8, 256, 256, 4, 2, 2, FORM_SLICE_K),
    BST_REG(AB_F16, 64, 64, 2, 2, FORM_SLICE_K),   BST_REG(AB_F16, 128, 128, 2, 2, FORM_SLICE_K),
    BST_DMA(AB_F16, 64, 64, 2, 2, 4, FORM_SLICE_K),  BST_DMA(AB_F16, 128, 128, 2, 2, 4, FORM_SLICE_K),
    BST_DMA(AB_F16, 256, 128, 2, 2, 3, FORM_SLICE_K),
    BST_REG(AB_BF16, 64, 64, 2, 2, FORM_SLICE_K),  BST_REG(AB_BF16, 128, 128, 2, 2, FORM_SLICE_K),
    BST_DMA(AB_BF16, 64, 64, 2, 2, 4, FORM_SLICE_K), BST_DMA(AB_BF16, 128, 128, 2, 2, 4, FORM_SLICE_K),
    BST_DMA(AB_BF16, 256, 128, 2, 2, 3, FORM_SLICE_K),
};

InstanceList instances_slicek() {
  return InstanceList{kList, (int)(sizeof(kList) / sizeof(kList[0]))};
}

}  // namespace bst
