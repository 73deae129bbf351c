// inst_mxfp8.hip -- compiled kernel instances for MX fp8 (e4m3 with e8m0 block scales) operands.
#include "bst_instances.hpp"

namespace bst {

static const Instance kList[] = {
    BST_REG(AB_MXE4M3, 64, 64, 2, 2, FORM_DENSE),  BST_REG(AB_MXE4M3, 128, 128, 2, 2, FORM_DENSE),
    BST_REG(AB_MXE4M3, 256, 128, 2, 2, FORM_DENSE), BST_REG(AB_MXE4M3, 256, 256, 4, 2, FORM_DENSE),
    BST_REG(AB_MXE4M3, 128, 64, 2, 2, FORM_DENSE),  BST_REG(AB_MXE4M3, 64, 128, 2, 2, FORM_DENSE),
    BST_DMA(AB_MXE4M3, 64, 64, 2, 2, 4, FORM_DENSE),  BST_DMA(AB_MXE4M3, 128, 128, 2, 2, 4, FORM_DENSE),
    BST_DMA(AB_MXE4M3, 256, 128, 2, 2, 3, FORM_DENSE), BST_DMA(AB_MXE4M3, 256, 256, 4, 2, 2, FORM_DENSE),
    BST_DMA(AB_MXE4M3, 128, 64, 2, 2, 4, FORM_DENSE),  BST_DMA(AB_MXE4M3, 64, 128, 2, 2, 4, FORM_DENSE),
    BST_DMA_ADD(AB_MXE4M3, 64, 128, 2, 2, 4), BST_DMA_ADD(AB_MXE4M3, 128, 128, 2, 2, 4),
    // two resident workgroups per CU, two stages
    BST_DMA_PAIR(AB_MXE4M3, 128, 128, 2, 2, 2, FORM_DENSE),
};

InstanceList instances_mxfp8() { return InstanceList{kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }

}  // namespace bst
