// inst_i8.hip -- compiled kernel instances for int8 operands.
#include "bst_instances.hpp"

namespace bst {

static const Instance kList[] = {
    BST_REG(AB_I8, 64, 64, 2, 2, FORM_DENSE),    BST_REG(AB_I8, 128, 128, 2, 2, FORM_DENSE),
    BST_REG(AB_I8, 256, 128, 2, 2, FORM_DENSE),  BST_REG(AB_I8, 256, 256, 4, 2, FORM_DENSE),
    BST_REG(AB_I8, 64, 64, 2, 2, FORM_SLICE_M),     BST_REG(AB_I8, 128, 128, 2, 2, FORM_SLICE_M),
    BST_REG(AB_I8, 256, 128, 2, 2, FORM_SLICE_M),   BST_REG(AB_I8, 256, 256, 4, 2, FORM_SLICE_M),
    BST_DMA(AB_I8, 64, 64, 2, 2, 4, FORM_DENSE),    BST_DMA(AB_I8, 128, 128, 2, 2, 4, FORM_DENSE),
    BST_DMA(AB_I8, 256, 128, 2, 2, 3, FORM_DENSE),  BST_DMA(AB_I8, 256, 256, 4, 2, 2, FORM_DENSE),
    BST_DMA(AB_I8, 64, 64, 2, 2, 4, FORM_SLICE_M),     BST_DMA(AB_I8, 128, 128, 2, 2, 4, FORM_SLICE_M),
    BST_DMA(AB_I8, 256, 128, 2, 2, 3, FORM_SLICE_M),   BST_DMA(AB_I8, 256, 256, 4, 2, 2, FORM_SLICE_M),
    BST_DMA_ADD(AB_I8, 128, 128, 2, 2, 4),
    // two resident workgroups per CU, two stages
    BST_DMA_PAIR(AB_I8, 128, 128, 2, 2, 2, FORM_DENSE),
    BST_DMA_PAIR(AB_I8, 128, 128, 2, 2, 2, FORM_SLICE_M),
};

InstanceList instances_i8() { return InstanceList{kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }

}  // namespace bst
