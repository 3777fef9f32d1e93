// Backward kernels (placeholder until implemented).
#include "ops.hpp"
#include "rotation.hpp"
namespace so2 {
int upload_generators_bwd(const float* host) { return upload_generators_here(host); }
int launch_edge_bwd(const Dims&, const GraphDev&, const float*, const float*, const float*, float*, float*, hipStream_t) { return hipErrorNotSupported; }
int launch_gate_bwd(const Dims&, long, const float*, const float*, float*, hipStream_t) { return hipErrorNotSupported; }
int launch_node_bwd(const Dims&, const GraphDev&, const float*, const float*, const float*, const float*, float*, float*, float*, float*, hipStream_t) { return hipErrorNotSupported; }
int launch_pos_grad(const GraphDev&, const float*, const float*, const float*, const float*, float*, float*, hipStream_t) { return hipErrorNotSupported; }
}
