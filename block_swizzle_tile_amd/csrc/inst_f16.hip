// inst_f16.hip -- compiled kernel instances for fp16 operands.
#include "bst_instances.hpp"

namespace bst {

static const Instance kList[] = {
    BST_REG(AB_F16, 64, 64, 2, 2, FORM_DENSE),   BST_REG(AB_F16, 128, 128, 2, 2, FORM_DENSE),
    BST_REG(AB_F16, 256, 128, 2, 2, FORM_DENSE), BST_REG(AB_F16, 128, 256, 2, 2, FORM_DENSE),
    BST_REG(AB_F16, 128, 192, 2, 2, FORM_DENSE), BST_REG(AB_F16, 128, 128, 2, 2, FORM_SLICE_M),
    BST_REG(AB_F16, 128, 64, 2, 2, FORM_DENSE),  BST_REG(AB_F16, 64, 128, 2, 2, FORM_DENSE),
    BST_REG(AB_F16, 256, 256, 4, 2, FORM_DENSE),
    BST_DMA(AB_F16, 64, 64, 2, 2, 4, FORM_DENSE),   BST_DMA(AB_F16, 128, 128, 2, 2, 4, FORM_DENSE),
    BST_DMA(AB_F16, 256, 128, 2, 2, 3, FORM_DENSE), BST_DMA(AB_F16, 128, 256, 2, 2, 3, FORM_DENSE),
    BST_DMA(AB_F16, 128, 192, 2, 2, 3, FORM_DENSE), BST_DMA(AB_F16, 128, 128, 2, 2, 4, FORM_SLICE_M),
    BST_DMA(AB_F16, 256, 256, 4, 2, 2, FORM_DENSE),
    BST_DMA(AB_F16, 128, 64, 2, 2, 4, FORM_DENSE),  BST_DMA(AB_F16, 64, 128, 2, 2, 4, FORM_DENSE),
    BST_DMA_ADD(AB_F16, 64, 64, 2, 2, 4), BST_DMA_ADD(AB_F16, 128, 128, 2, 2, 4),
    // two resident workgroups per CU, two stages
    BST_DMA_PAIR(AB_F16, 128, 128, 2, 2, 2, FORM_DENSE),
    BST_DMA_PAIR(AB_F16, 128, 128, 2, 2, 2, FORM_SLICE_M),
};

InstanceList instances_f16() { return InstanceList{kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }

}  // namespace bst
