// inst_f16.hip -- compiled kernel instances for fp16 operands.
#include "bst_instances.hpp"

namespace bst {

static const Instance kList[] = {
    BST_REG(AB_F16, 64, 64, 2, 2, false),   BST_REG(AB_F16, 128, 128, 2, 2, false),
    BST_REG(AB_F16, 256, 128, 2, 2, false), BST_REG(AB_F16, 128, 256, 2, 2, false),
    BST_REG(AB_F16, 128, 192, 2, 2, false), BST_REG(AB_F16, 128, 128, 2, 2, true),
    BST_REG(AB_F16, 128, 64, 2, 2, false),  BST_REG(AB_F16, 64, 128, 2, 2, false),
    BST_REG(AB_F16, 256, 256, 4, 2, false),
    BST_DMA(AB_F16, 64, 64, 2, 2, 4, false),   BST_DMA(AB_F16, 128, 128, 2, 2, 4, false),
    BST_DMA(AB_F16, 256, 128, 2, 2, 3, false), BST_DMA(AB_F16, 128, 256, 2, 2, 3, false),
    BST_DMA(AB_F16, 128, 192, 2, 2, 3, false), BST_DMA(AB_F16, 128, 128, 2, 2, 4, true),
    BST_DMA(AB_F16, 256, 256, 4, 2, 2, false),
    BST_DMA(AB_F16, 128, 64, 2, 2, 4, false),  BST_DMA(AB_F16, 64, 128, 2, 2, 4, false),
    BST_DMA_ADD(AB_F16, 64, 64, 2, 2, 4), BST_DMA_ADD(AB_F16, 128, 128, 2, 2, 4),
};

InstanceList instances_f16() { return InstanceList{kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }

}  // namespace bst
