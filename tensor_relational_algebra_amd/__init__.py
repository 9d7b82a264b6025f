"""MI355X-native executor for extended EinSum as tensor-relational algebra."""
