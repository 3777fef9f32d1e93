// Double-backward kernels (placeholder until implemented).
#include "ops.hpp"
#include "rotation.hpp"
namespace so2 {
int upload_generators_dual(const float* host) { return upload_generators_here(host); }
int launch_edge_dual(const Dims&, const GraphDev&, const float*, const float*, const float*, const float*, const float*, const float*, const float*, float*, float*, hipStream_t) { return hipErrorNotSupported; }
int launch_gate_dual(const Dims&, long, const float*, const float*, float*, hipStream_t) { return hipErrorNotSupported; }
int launch_node_dual(const Dims&, const GraphDev&, const float*, const float*, const float*, const float*, float*, hipStream_t) { return hipErrorNotSupported; }
int launch_edge_bwd_dual(const Dims&, const GraphDev&, const float*, const float*, const float*, float*, hipStream_t) { return hipErrorNotSupported; }
int launch_gate_dbwd(const Dims&, long, const float*, const float*, const float*, float*, hipStream_t) { return hipErrorNotSupported; }
int launch_node_bwd_dual(const Dims&, const GraphDev&, const float*, const float*, const float*, const float*, const float*, const float*, const float*, float*, float*, float*, hipStream_t) { return hipErrorNotSupported; }
}
